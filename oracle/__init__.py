"""CPU oracle for the block-quantized matmul: TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import or run anything in this
package.  The product path (the HIP library and its Python binding) never
imports it and shares no code, table or helper with it.

What is here:

* ``mq_oracle``     -- plain numpy (f64 / int64) definitions of what the hot
                       path computes: block decoders, the activation
                       quantizer, the GEMV, the int block dots and the MMQ
                       product.
  ``repack`` / ``unpack_repacked`` define the repacked weight layout;
                       ``q4_k_plane`` / ``act_f6_section`` the fp6 planes of the
                       Q4_K prefill product (weights and activations);
                       ``q4_k_row_tiled`` Q4_K's row-tiled layout for the
                       long-row GEMV.
* ``bitwise_decode`` -- a second, independently written per-block decoder that
                       assembles every field bit by bit; it exists only to
                       cross-check ``mq_oracle``'s vectorised decoders.

Pinning status (each function's docstring repeats it):

* The arithmetic of every function is pinned by tests that do not retype it:
  hand-worked blocks with closed-form values, a brute-force product in exact
  rationals, closed forms, invariants and planted-mistake (mutation) checks.
* The *bit layouts* of every type are the public GGUF layouts; the pages state
  only block byte sizes (Q8_0, Q4_K, Q4_0, Q5_K) and the list of types.  Agreement with real GGUF files is
  **parity unpinned**: no GGUF file exists in this environment to pin it.
"""

from .mq_oracle import (  # noqa: F401
    Q4_0, Q4_1, Q5_0, Q5_1, Q8_0, Q4_K, Q5_K, Q6_K, BLOCK_VALUES, BLOCK_BYTES, LEGACY,
    f16_bits_to_f64, row_bytes,
    q8_0_fields, q4_k_fields, q5_k_fields, q6_k_fields, legacy_fields, decode,
    gemv, quantize_act, block_dots, mmq, mmq_from_block_dots,
    REPACK_SLOT, repack, unpack_repacked,
    PLANE_ROWS, ACT_PLANE_ROWS, e2m3_value, e2m3_code_of_half, fp6_records, bf16_hilo, q4_k_plane,
    act_f6_section, row_tile_rows, q4_k_row_tiled, unpack_q4_k_row_tiled,
)
