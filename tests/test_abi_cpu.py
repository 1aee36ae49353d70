"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, computes sizes, and refuses bad arguments before any HIP call.

No kernel is launched here (this machine may have no GPU): every call that
passes validation would need mq_init, and the refusals tested below happen
first.
"""

import ctypes
import os
import re

import pytest

from block_quantized_matmul_mq_amd import mq

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mq.h")
FAKE = 0x10000  # a 256-byte aligned non-null pointer value that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mq_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = mq.load()
    names = declared_functions()
    assert "mq_gemv" in names and "mq_gemm" in names and "mq_quantize_act" in names
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(mq._SIGNATURES), "binding and header disagree"


def test_weight_bytes_are_exact_payload_sizes():
    assert mq.weight_bytes(mq.Q4_K, 18944, 3584) == 38191104
    assert mq.weight_bytes(mq.Q4_K, 3584, 18944) == 38191104
    assert mq.weight_bytes(mq.Q6_K, 152064, 3584) == 447068160
    assert mq.weight_bytes(mq.Q8_0, 4864, 896) == 4630528
    assert mq.weight_bytes(mq.Q4_K, 10, 100) == 0      # K not a whole super-block
    assert mq.weight_bytes(99, 10, 256) == 0           # unknown type
    assert mq.weight_bytes(mq.Q8_0, 0, 32) == 0
    # the 32-value types and Q5_K (block bytes 18, 20, 22, 24 per 32 values and 176 per 256)
    assert mq.weight_bytes(mq.Q4_0, 4864, 896) == 4864 * 28 * 18
    assert mq.weight_bytes(mq.Q4_1, 4864, 896) == 4864 * 28 * 20
    assert mq.weight_bytes(mq.Q5_0, 4864, 896) == 4864 * 28 * 22
    assert mq.weight_bytes(mq.Q5_1, 4864, 896) == 4864 * 28 * 24
    assert mq.weight_bytes(mq.Q5_K, 18944, 3584) == 18944 * 14 * 176
    assert mq.weight_bytes(mq.Q5_K, 10, 100) == 0
    assert mq.weight_bytes(mq.Q4_0, 10, 48) == 0       # K not a whole 32-value block
    # no repacked layout for them
    for t in (mq.Q4_0, mq.Q4_1, mq.Q5_0, mq.Q5_1, mq.Q5_K):
        assert mq.weight_bytes(t | mq.REPACKED, 10, 256) == 0


@pytest.mark.parametrize("M,K", [(37, 96), (5, 128), (1, 32)])
def test_activation_plane_layout(M, K):
    total, so, uo = mq.act_layout(M, K)
    fo = mq.load().mq_act_f6_offset(M, K)
    T = (K + 63) // 64     # 64-value steps, the last one half empty when K % 64 == 32
    Mp = -(-M // 128) * 128   # the fp6 section's rows, padded with zero rows
    assert so >= M * K and so % 256 == 0
    assert uo >= so + 4 * M * (K // 32) and uo % 256 == 0
    assert fo >= uo + 4 * M * (K // 32) and fo % 256 == 0
    assert total == fo + 128 * Mp * T
    assert mq.act_bytes(M, 100) == 0
    assert mq.load().mq_act_f6_offset(M, 100) == 0


def _rc(fn, *args):
    return fn(*args)


def test_quantize_act_refusals():
    lib = mq.load()
    assert lib.mq_quantize_act(None, FAKE, 4, 64, None) == -1
    assert lib.mq_quantize_act(FAKE, FAKE, 0, 64, None) == -1
    assert lib.mq_quantize_act(FAKE, FAKE, 4, 48, None) == -2
    assert "multiple of 32" in mq.last_error()
    assert lib.mq_quantize_act(FAKE + 4, FAKE, 4, 64, None) == -5
    assert lib.mq_quantize_act(FAKE, FAKE + 16, 4, 64, None) == -5
    assert lib.mq_quantize_act(FAKE, FAKE, 4, 1 << 16, None) == -2


def test_gemv_refusals():
    lib = mq.load()
    assert lib.mq_gemv(None, mq.Q4_K, FAKE, FAKE, 8, 256, None) == -1
    assert lib.mq_gemv(FAKE, 10, FAKE, FAKE, 8, 256, None) == -3       # q2_K is not served here
    assert "unsupported weight type 10" in mq.last_error()
    assert lib.mq_gemv(FAKE, mq.Q4_K, FAKE, FAKE, 8, 128, None) == -2  # K % 256
    assert "K=128" in mq.last_error()
    assert lib.mq_gemv(FAKE, mq.Q8_0, FAKE, FAKE, 8, 48, None) == -2   # K % 32
    assert lib.mq_gemv(FAKE, mq.Q8_0, FAKE, FAKE, -1, 64, None) == -1
    assert lib.mq_gemv(FAKE + 2, mq.Q8_0, FAKE, FAKE, 8, 64, None) == -5
    assert lib.mq_gemv(FAKE, mq.Q8_0, FAKE + 8, FAKE, 8, 64, None) == -5
    assert lib.mq_gemv(FAKE, mq.Q8_0, FAKE, FAKE + 2, 8, 64, None) == -5


def test_gemm_refusals():
    lib = mq.load()
    assert lib.mq_gemm(FAKE, mq.Q4_K, FAKE, None, 4, 8, 256, None, 0, None) == -1
    assert lib.mq_gemm(FAKE, mq.Q4_K, FAKE, FAKE, 0, 8, 256, None, 0, None) == -1
    assert lib.mq_gemm(FAKE, mq.Q6_K, FAKE, FAKE, 4, 8, 96, None, 0, None) == -2
    assert lib.mq_gemm(FAKE, 11, FAKE, FAKE, 4, 8, 256, None, 0, None) == -3   # q3_K
    assert lib.mq_gemm(FAKE, mq.Q4_K, FAKE + 16, FAKE, 4, 8, 256, None, 0, None) == -5
    assert lib.mq_debug_gemm_blockdots(FAKE, mq.Q4_K, FAKE, None, 4, 8, 256, None) == -1


def test_gemm_scratch_is_sized_by_the_split_plan():
    tile = 128 * 128 * 4

    def sk(tiles, pieces, tile_bytes=tile):
        # 1 KiB of uint32 counters (at most 256 cut tiles), then the partial slots
        return 1024 + tiles * pieces * tile_bytes

    # Q4_K's MMQ plane runs the fp6 kernel: 128 x 128 tiles, two workgroups per CU (rounds
    # of 512), 64-value K-steps, at least 4 per range, ranges for half a round (one workgroup
    # per CU); the counters, then partial tiles of 128 x 128 f32.
    P = mq.Q4_K | mq.REPACKED
    # 512 tiles fill one round: no split, no scratch
    assert mq.gemm_scratch_bytes(P, 512, 16384, 3584) == 0
    # 592 tiles: 512 whole, the last 80 cut into 3 K ranges
    assert mq.gemm_scratch_bytes(P, 512, 18944, 3584) == sk(80, 3)
    # a last round more than half full is not cut (2400 tiles: 352 in the last round)
    assert mq.gemm_scratch_bytes(P, 512 * 3, 128 * 200, 3584) == 0
    # 612 tiles: the last 100 cut into 2 ranges; 70 tiles into 3 (56 steps: uneven); 140
    # tiles would get one range each for 256 workgroups: none is cut
    assert mq.gemm_scratch_bytes(P, 100, 306 * 256 - 13, 3584) == sk(100, 2)
    assert mq.gemm_scratch_bytes(P, 100, 70 * 128, 3584) == sk(70, 3)
    assert mq.gemm_scratch_bytes(P, 100, 140 * 128, 3584) == 0
    # any M, small ones included (two tiles of 128 x 128, 56 steps: 14 ranges)
    assert mq.gemm_scratch_bytes(P, 1, 256, 3584) == sk(2, 14)
    # the int8 kernel (every type on the GGUF layout): 128 x 128 tiles in rounds of 512
    # workgroups (two per CU), 128-value K-steps, at least 2 per range, ranges for half a
    # round (one workgroup per CU); the counters, then the partial tiles.  The 7B ffn_up
    # product has 592 tiles: 512 whole, the last 80 cut into 3.
    t32 = 32 * 128 * 4
    assert mq.gemm_scratch_bytes(mq.Q4_K, 512, 18944, 3584) == sk(80, 3)
    # at most 256 tiles of 128 rows: 32-row tiles instead.  512 x 512 has 64 of them, cut
    # into ranges for 256 workgroups (one per CU): 4 each
    for t in (mq.Q8_0, mq.Q6_K, mq.Q5_K, mq.Q4_0, mq.Q4_1, mq.Q5_0, mq.Q5_1):
        assert mq.gemm_scratch_bytes(t, 512, 512, 3584) == sk(64, 4, t32)
    # Q4_K there runs the kernel with one 32 x 32 tile per workgroup and the K range split
    # over its waves: no scratch.  It is taken while its waves run at most 5 K-steps more
    # than the int8 kernel's ranges: at 20 x 3000 x 3584 (7 against 3) and at
    # 40 x 100 x 8192 (16 against 2) it is not.
    assert mq.gemm_scratch_bytes(mq.Q4_K, 512, 512, 3584) == 0
    assert mq.gemm_scratch_bytes(mq.Q4_K, 1024, 1024, 3584) == 0
    assert mq.gemm_scratch_bytes(mq.Q4_K, 20, 3000, 32768) == sk(24, 10, t32)
    assert mq.gemm_scratch_bytes(mq.Q4_K, 40, 100, 8192) == sk(2, 32, t32)
    # 448 32-row tiles (a last round more than half full): nothing cut
    assert mq.gemm_scratch_bytes(mq.Q4_K, 512, 3584, 3584) == 0
    assert mq.gemm_scratch_bytes(mq.Q4_K, 2048, 1024, 5120) == 0
    # 257 tiles of 128 rows stay 128-row tiles: 257 in one round, nothing cut
    assert mq.gemm_scratch_bytes(mq.Q4_K, 40, 128 * 257, 3584) == 0
    # 8 < M <= 32: 32 x 128 tiles; the vocab head at M = 9 has 1188 of them, and its last
    # 164 would get one range each: none is cut.  At M = 20 and N = 3000, 24 tiles get 10
    # (Q8_0; Q4_K runs the split-over-waves kernel there).
    assert mq.gemm_scratch_bytes(mq.Q6_K, 9, 152064, 3584) == 0
    assert mq.gemm_scratch_bytes(mq.Q4_K, 9, 152064, 3584) == 0
    assert mq.gemm_scratch_bytes(mq.Q8_0, 20, 3000, 3584) == sk(24, 10, t32)
    assert mq.gemm_scratch_bytes(mq.Q4_K, 20, 3000, 3584) == 0
    # M <= 8: the multi-row GEMV, no scratch -- unless the rows do not fit its LDS
    assert mq.gemm_scratch_bytes(mq.Q6_K, 8, 152064, 3584) == 0
    assert mq.gemm_scratch_bytes(mq.Q6_K, 8, 260, 32768) > 0
    # invalid shapes report 0 (the call itself refuses them)
    assert mq.gemm_scratch_bytes(mq.Q4_K, 512, 512, 100) == 0
    assert mq.gemm_scratch_bytes(99, 512, 512, 3584) == 0
    lib = mq.load()
    need = mq.gemm_scratch_bytes(mq.Q8_0, 512, 512, 3584)
    assert lib.mq_gemm(FAKE, mq.Q8_0, FAKE, FAKE, 512, 512, 3584, None, 0, None) == -4
    assert "required" in mq.last_error()
    assert lib.mq_gemm(FAKE, mq.Q8_0, FAKE, FAKE, 512, 512, 3584, FAKE, need - 4, None) == -4
    assert lib.mq_gemm(FAKE, mq.Q8_0, FAKE, FAKE, 512, 512, 3584, FAKE + 4, need, None) == -5
    # a product that needs no scratch takes none
    assert mq.gemm_scratch_bytes(mq.Q4_K, 512, 512, 3584) == 0


def test_repacked_sizes_and_type_flag():
    R = mq.REPACKED
    assert mq.repack_bytes(mq.Q6_K, 152064, 3584) == 152064 * 14 * 224
    assert mq.repack_bytes(mq.Q8_0, 4864, 896) == 4864 * 28 * 36
    assert mq.weight_bytes(mq.Q6_K | R, 10, 512) == 10 * 2 * 224
    assert mq.weight_bytes(mq.Q8_0 | R, 10, 64) == 10 * 2 * 36
    # Q4_K: the MMQ plane, 80 bytes per 64-value step per row, rows padded to 256
    assert mq.repack_bytes(mq.Q4_K, 18944, 3584) == 56 * 80 * 18944
    assert mq.repack_bytes(mq.Q4_K, 10, 256) == 4 * 80 * 256
    assert mq.weight_bytes(mq.Q4_K | R, 300, 512) == 8 * 80 * 512
    assert mq.repack_bytes(mq.Q4_K, 10, 128) == 0
    assert mq.repack_bytes(mq.Q6_K | R, 10, 256) == 0
    assert mq.repack_bytes(mq.Q6_K, 10, 100) == 0
    assert mq.gemm_scratch_bytes(mq.Q6_K | R, 9, 152064, 3584) == mq.gemm_scratch_bytes(mq.Q6_K, 9, 152064, 3584)


def test_row_tiled_sizes_and_refusals():
    """Q4_K's row-tiled layout (MQ_ROW_TILED): the byte counts the library reports equal
    the oracle's layout; it exists for Q4_K rows of more than 16 super-blocks only; only
    mq_gemv reads it."""
    import numpy as np
    import oracle
    from block_quantized_matmul_mq_amd import synth
    T = mq.Q4_K | mq.ROW_TILED
    assert mq.weight_bytes(T, 3584, 18944) == mq.weight_bytes(mq.Q4_K, 3584, 18944) == 38191104
    for N, K in [(3, 17 * 256), (301, 17 * 256), (513, 18 * 256), (5000, 20 * 256)]:
        raw = synth.random_blocks(oracle.Q4_K, N, K, np.random.default_rng(N)).reshape(-1)
        assert mq.repack_bytes(T, N, K) == mq.weight_bytes(T, N, K) == oracle.q4_k_row_tiled(raw, N, K).size
    assert mq.weight_bytes(T, 3584, 4096) == 0                      # 16 super-blocks: not a long row
    assert mq.weight_bytes(mq.Q6_K | mq.ROW_TILED, 3584, 18944) == 0
    assert mq.weight_bytes(T | mq.REPACKED, 3584, 18944) == 0
    assert mq.gemm_scratch_bytes(T, 512, 3584, 18944) == 0
    lib = mq.load()
    far = FAKE + (1 << 28)
    nb = mq.weight_bytes(mq.Q4_K, 300, 4352)
    rb = mq.repack_bytes(T, 300, 4352)
    assert lib.mq_repack(FAKE, mq.Q6_K | mq.ROW_TILED, 300, 4352, nb, far, rb, None) == -3
    assert lib.mq_repack(FAKE, T, 300, 4096, mq.weight_bytes(mq.Q4_K, 300, 4096), far, rb, None) == -2
    assert "more than 16 super-blocks" in mq.last_error()
    assert lib.mq_repack(FAKE, T, 300, 4352, nb - 144, far, rb, None) == -4          # exact input length
    assert lib.mq_repack(FAKE, T, 300, 4352, nb, far, rb - 1, None) == -4
    assert lib.mq_gemv(FAKE, T, FAKE, FAKE, 300, 4096, None) == -2
    assert lib.mq_gemv(FAKE, mq.Q6_K | mq.ROW_TILED, FAKE, FAKE, 300, 4352, None) == -3
    assert lib.mq_gemm(FAKE, T, FAKE, FAKE, 40, 300, 4352, None, 0, None) == -3
    assert "only mq_gemv reads" in mq.last_error()
    assert lib.mq_debug_gemm_blockdots(FAKE, T, FAKE, FAKE, 40, 300, 4352, None) == -3


def test_repack_refusals():
    lib = mq.load()
    nb6 = mq.weight_bytes(mq.Q6_K, 8, 512)
    rb6 = mq.repack_bytes(mq.Q6_K, 8, 512)
    far = FAKE + (1 << 24)
    assert lib.mq_repack(None, mq.Q6_K, 8, 512, nb6, far, rb6, None) == -1
    assert lib.mq_repack(FAKE, mq.Q5_K, 8, 512, mq.weight_bytes(mq.Q5_K, 8, 512), far, 1 << 20, None) == -3
    assert "no repacked layout" in mq.last_error()
    nb4 = mq.weight_bytes(mq.Q4_K, 8, 512)
    assert lib.mq_repack(FAKE, mq.Q4_K, 8, 512, nb4 - 144, far, 1 << 20, None) == -4     # exact length only
    assert lib.mq_repack(FAKE, mq.Q4_K, 8, 512, nb4, far, mq.repack_bytes(mq.Q4_K, 8, 512) - 1, None) == -4
    assert lib.mq_repack(FAKE, mq.Q6_K | mq.REPACKED, 8, 512, nb6, far, rb6, None) == -3
    assert lib.mq_repack(FAKE, mq.Q6_K, 8, 500, nb6, far, rb6, None) == -2
    assert lib.mq_repack(FAKE, mq.Q6_K, 8, 512, nb6 + 1, far, rb6, None) == -4      # exact length only
    assert "exactly" in mq.last_error()
    assert lib.mq_repack(FAKE, mq.Q6_K, 8, 512, nb6, far, rb6 - 1, None) == -4
    assert lib.mq_repack(FAKE + 2, mq.Q6_K, 8, 512, nb6, far, rb6, None) == -5
    assert lib.mq_repack(FAKE, mq.Q6_K, 8, 512, nb6, FAKE + 16, rb6, None) == -1    # overlap
    assert "overlap" in mq.last_error()
    assert lib.mq_gemv(FAKE, mq.Q4_K | mq.REPACKED, FAKE, FAKE, 8, 256, None) == -3   # the plane is for mq_gemm
    assert "only mq_gemm reads" in mq.last_error()


def test_calls_without_init_are_refused_not_run():
    # Valid arguments but mq_init has not succeeded (and there may be no device
    # at all): the call must return an error code, never launch.
    lib = mq.load()
    rc = lib.mq_gemv(FAKE, mq.Q4_K, FAKE, FAKE, 8, 256, None)
    assert rc in (-6, -8)
    assert mq.last_error().startswith("mq_gemv")


def test_init_refuses_a_bad_device_index():
    lib = mq.load()
    assert lib.mq_init(-1) == -1
    assert lib.mq_init(10 ** 6) == -1


def _refused(code, fn, *args, **kw):
    with pytest.raises(mq.MQError) as ei:
        fn(*args, **kw)
    assert ei.value.code == code, str(ei.value)
    return str(ei.value)


def test_binding_refuses_bad_tensors_before_any_call():
    """The binding checks every tensor against the call's sizes, dtypes, contiguity and
    device before handing its pointer to the library (the C ABI takes no lengths for W,
    x, Xq or Y, so a mismatch would otherwise read or write past a buffer)."""
    import torch
    N, K, M = 8, 256, 3
    W = torch.zeros(mq.weight_bytes(mq.Q4_K, N, K), dtype=torch.uint8)
    x = torch.zeros(K)
    # GEMV: exact payload length, x f32 of K, y f32 of N, contiguity, then the device
    assert "exactly 1152" in _refused(-4, mq.gemv, W[:-1], mq.Q4_K, x, N, K)
    _refused(-4, mq.gemv, torch.zeros(len(W) + 16, dtype=torch.uint8), mq.Q4_K, x, N, K)
    _refused(-3, mq.gemv, W, mq.Q4_K, x, N, 100)                       # K not a whole block
    _refused(-1, mq.gemv, W, mq.Q4_K, x.double(), N, K)
    _refused(-1, mq.gemv, W, mq.Q4_K, x.half(), N, K)
    _refused(-4, mq.gemv, W, mq.Q4_K, x[:-1], N, K)
    _refused(-1, mq.gemv, W, mq.Q4_K, torch.zeros(2 * K)[::2], N, K)   # strided x
    _refused(-4, mq.gemv, W, mq.Q4_K, x, N, K, y=torch.zeros(N - 1))
    _refused(-1, mq.gemv, W, mq.Q4_K, x, N, K, y=torch.zeros(N, dtype=torch.float64))
    assert "one GPU device" in _refused(-6, mq.gemv, W, mq.Q4_K, x, N, K, y=torch.zeros(N))
    # quantize_act: 2-D f32 X, K a multiple of 32, Xq large enough
    X = torch.zeros(M, K)
    _refused(-1, mq.quantize_act, X.reshape(-1))
    _refused(-1, mq.quantize_act, X.double())
    _refused(-1, mq.quantize_act, X.t())
    _refused(-2, mq.quantize_act, torch.zeros(M, 48))
    _refused(-4, mq.quantize_act, X, Xq=torch.zeros(mq.act_bytes(M, K) - 1, dtype=torch.uint8))
    _refused(-6, mq.quantize_act, X, Xq=torch.zeros(mq.act_bytes(M, K), dtype=torch.uint8))
    # GEMM and the block-dot export: the plane of M x K, Y f32 of M x N, D int32 of M x N x G
    Xq = torch.zeros(mq.act_bytes(M, K), dtype=torch.uint8)
    _refused(-4, mq.gemm, W[:-1], mq.Q4_K, Xq, M, N, K)
    _refused(-4, mq.gemm, W, mq.Q4_K, Xq[:-1], M, N, K)
    _refused(-4, mq.gemm, W, mq.Q4_K, Xq, M + 1, N, K)                 # plane of fewer rows
    _refused(-4, mq.gemm, W, mq.Q4_K, Xq, M, N, K, Y=torch.zeros(M, N - 1))
    _refused(-1, mq.gemm, W, mq.Q4_K, Xq, M, N, K, Y=torch.zeros(N, M).t())
    _refused(-6, mq.gemm, W, mq.Q4_K, Xq, M, N, K, Y=torch.zeros(M, N))
    _refused(-1, mq.gemm_blockdots, W, mq.Q4_K, Xq, M, N, K, D=torch.zeros(M, N, K // 32))
    _refused(-4, mq.gemm_blockdots, W, mq.Q4_K, Xq, M, N, K, D=torch.zeros(M, N, 1, dtype=torch.int32))
    # repack: exact payload, output large enough
    W6 = torch.zeros(mq.weight_bytes(mq.Q6_K, N, K), dtype=torch.uint8)
    _refused(-4, mq.repack, W6[:-2], mq.Q6_K, N, K)
    _refused(-4, mq.repack, W6, mq.Q6_K, N, K, Wr=torch.zeros(mq.repack_bytes(mq.Q6_K, N, K) - 1,
                                                                dtype=torch.uint8))
