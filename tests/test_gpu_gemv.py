"""GPU parity of mq_gemv (f32 activation) against the oracle's f64 GEMV."""

import numpy as np
import pytest

import oracle
from block_quantized_matmul_mq_amd import mq, synth

from gpu_cases import ALL_TYPES, BLOCK, NAMES, check_normalized, device, row_norms, say, to_dev, weights

pytestmark = pytest.mark.gpu

TYPES = ALL_TYPES


def run_gemv(raw, qtype, x, N, K, rows=None, what=""):
    import torch
    dev = device()
    say(f"gemv {NAMES[qtype]} N={N} K={K} {what}")
    W = to_dev(raw.reshape(-1), dev)
    y = mq.gemv(W, qtype, to_dev(x, dev), N, K)
    torch.cuda.synchronize()
    assert mq.last_kernel().startswith("gemv")
    y = y.cpu().numpy()
    rows = np.arange(N) if rows is None else rows
    sub = raw.reshape(N, -1)[rows]
    y_ref = oracle.gemv(sub, qtype, x, len(rows), K)
    wn = row_norms(raw, qtype, N, K, rows)
    xn = np.array([np.linalg.norm(x.astype(np.float64))])
    return check_normalized(y[rows][None, :], y_ref[None, :], wn, xn, f"{NAMES[qtype]} {N}x{K} {what}")


def small_shapes(qtype):
    b = BLOCK[qtype]
    # one block, several K-steps with a ragged last step, ragged N tails
    return [(1, b), (5, b), (37, 2 * b), (130, 2048 + b), (300, 4096), (67, 8192 + 3 * b)]


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
@pytest.mark.parametrize("kind", ["quantized", "random"])
def test_gemv_small_and_ragged(qtype, kind):
    for i, (N, K) in enumerate(small_shapes(qtype)):
        raw = weights(qtype, N, K, kind, i)
        x = synth.activations(1, K, config_index=10, tensor_index=i)[0]
        run_gemv(raw, qtype, x, N, K, what=kind)


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
def test_gemv_zero_rows_and_zero_input(qtype):
    N, K = 20, 2 * BLOCK[qtype]
    raw = weights(qtype, N, K, "quantized", 3)
    raw = raw.reshape(N, -1).copy()
    raw[4] = 0
    raw[11] = 0
    x = synth.activations(1, K, config_index=11, tensor_index=0)[0]
    run_gemv(raw, qtype, x, N, K, what="zero rows")
    run_gemv(raw, qtype, np.zeros(K, np.float32), N, K, what="zero x")


def test_gemv_q8_0_config1_ffn_up():
    N, K = 4864, 896
    raw = synth.quantized_weight(mq.Q8_0, N, K, 0, 0)
    x = synth.activations(1, K, config_index=0)[0]
    run_gemv(raw, mq.Q8_0, x, N, K, what="0.5B ffn_up")


def test_gemv_q8_0_7b_shape():
    N, K = 18944, 3584
    raw = synth.quantized_weight(mq.Q8_0, N, K, 0, 5)
    x = synth.activations(1, K, config_index=0, tensor_index=5)[0]
    run_gemv(raw, mq.Q8_0, x, N, K, what="7B ffn_up shape")


@pytest.mark.parametrize("N,K,tensor", [(18944, 3584, 0), (3584, 18944, 1)], ids=["ffn_up", "ffn_down"])
def test_gemv_q4_k_config2(N, K, tensor):
    raw = synth.quantized_weight(mq.Q4_K, N, K, 1, tensor)
    x = synth.activations(1, K, config_index=1, tensor_index=tensor)[0]
    run_gemv(raw, mq.Q4_K, x, N, K, what="7B FFN")


def test_gemv_q6_k_config3_head_sampled():
    N, K = 152064, 3584
    raw = synth.quantized_weight(mq.Q6_K, N, K, 2, 0)
    x = synth.activations(1, K, config_index=2)[0]
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.integers(0, N, 3000), np.arange(64), np.arange(N - 64, N)]))
    run_gemv(raw, mq.Q6_K, x, N, K, rows=rows, what="vocab head (sampled rows)")


@pytest.mark.parametrize("qtype,N,K,tensor", [(mq.Q4_K, 5120, 5120, 0), (mq.Q4_K, 1024, 5120, 1),
                                              (mq.Q4_K, 13824, 5120, 2), (mq.Q6_K, 5120, 13824, 3)],
                         ids=["attn_q", "attn_k", "ffn_up", "ffn_down"])
def test_gemv_config5_14b(qtype, N, K, tensor):
    raw = synth.quantized_weight(qtype, N, K, 4, tensor)
    x = synth.activations(1, K, config_index=4, tensor_index=tensor)[0]
    rows = None if N * K <= 5120 * 5120 else np.random.default_rng(1).choice(N, 2048, replace=False)
    run_gemv(raw, qtype, x, N, K, rows=rows, what="14B")


@pytest.mark.parametrize("N,K,kind,sampled", [(16384 + 77, 3072, "random", False),
                                              (20000, 3584, "quantized", False),
                                              (2 * 16384 + 5, 4096, "random", False),
                                              (8192, 3584, "quantized", False),
                                              (65536 - 3, 3584, "random", True)],
                         ids=["ragged_K3072", "K3584", "K4096_ring_wraps", "two_tiles_per_cu",
                              "sixteen_tiles_per_cu"])
def test_gemv_q4_k_wide_matrix_core_path(N, K, kind, sampled):
    """Wide Q4_K matrices (at least two 16-row tiles per CU, 12 to 16 super-blocks per row)
    take the int8 matrix-core kernel: a ragged last tile, idle waves (K < 4096), tiles per
    workgroup below the prefetch depth, ring wrap-around with a tail, the largest tile
    count per workgroup, and an x with all-zero and tiny blocks."""
    raw = weights(mq.Q4_K, N, K, kind, 7)
    x = synth.activations(1, K, config_index=10, tensor_index=N % 97)[0]
    x[32:64] = 0.0
    x[96:128] *= 1e-30
    rows = None
    if sampled:
        rng = np.random.default_rng(N)
        rows = np.unique(np.concatenate([rng.integers(0, N, 3000), np.arange(32), np.arange(N - 32, N)]))
    run_gemv(raw, mq.Q4_K, x, N, K, rows=rows, what=f"{kind} matrix-core")
    assert "mfma" in mq.last_kernel()


@pytest.mark.parametrize("N,K,kind", [(3584 - 5, 18944, "random"),
                                      (2048 + 3, 13824, "quantized"),
                                      (4096, 14336, "random"),
                                      (3000, 256 * 17, "quantized"),
                                      (2304, 24576, "random")],
                         ids=["ragged_7b_down", "nine_row_tiles", "sixteen_row_tiles", "seventeen_super_blocks",
                              "longest_rows"])
def test_gemv_q4_k_long_row_matrix_core_path(N, K, kind):
    """Long Q4_K rows (more than 16 super-blocks) at 8 to 16 rows per CU take the
    long-row matrix-core kernel: a short last tile, tiles of 9 and 16 rows, waves with
    one and two items (17 super-blocks), the largest K the kernel stages, and an x with
    all-zero and tiny blocks."""
    raw = weights(mq.Q4_K, N, K, kind, 8)
    x = synth.activations(1, K, config_index=10, tensor_index=N % 89)[0]
    x[32:64] = 0.0
    x[K - 96:K - 64] *= 1e-30
    run_gemv(raw, mq.Q4_K, x, N, K, what=f"{kind} long-row matrix-core")
    assert "mfma_long" in mq.last_kernel()


@pytest.mark.parametrize("N,K,kind,sampled", [(16 * 512 + 4, 3584, "random", False),
                                              (9000, 3072, "quantized", False),
                                              (8192 + 16 * 37, 4096, "random", False),
                                              (8192 + 8 * 11, 3328, "random", False),
                                              (152064, 3584, "quantized", True)],
                         ids=["ragged_tile_K3584", "twelve_super_blocks", "sixteen_super_blocks",
                              "odd_row_alignment", "vocab_head"])
def test_gemv_q6_k_matrix_core_path(N, K, kind, sampled):
    """Wide Q6_K matrices in the GGUF layout (at least two 16-row tiles per CU, 12 to 16
    super-blocks per row, the matrix ending on a 16-byte boundary) take the whole-tile
    matrix-core kernel: a ragged last tile, idle waves (K = 3072), every wave busy
    (K = 4096), rows of 13 super-blocks (2730 bytes: odd rows start 2 bytes off a dword,
    so the lanes of one MFMA realign by different amounts), the vocab head, and an x with
    all-zero and tiny blocks and runs."""
    raw = weights(mq.Q6_K, N, K, kind, 9)
    x = synth.activations(1, K, config_index=10, tensor_index=N % 83)[0]
    x[32:64] = 0.0
    x[112:128] *= 1e-30
    rows = None
    if sampled:
        rng = np.random.default_rng(N)
        rows = np.unique(np.concatenate([rng.integers(0, N, 3000), np.arange(32), np.arange(N - 32, N)]))
    run_gemv(raw, mq.Q6_K, x, N, K, rows=rows, what=f"{kind} matrix-core")
    assert mq.last_kernel() == "gemv_mfma<q6_K>"


def test_gemv_q6_k_unaligned_end_takes_the_vector_kernel():
    # 8193 rows of 2940 bytes do not end on a 16-byte boundary: the vector kernel runs
    N, K = 8193, 3584
    raw = weights(mq.Q6_K, N, K, "quantized", 10)
    x = synth.activations(1, K, config_index=10, tensor_index=3)[0]
    run_gemv(raw, mq.Q6_K, x, N, K, what="unaligned end")
    assert mq.last_kernel() == "gemv<q6_K>"



WIDE = [mq.Q8_0, mq.Q4_0, mq.Q5_0]


@pytest.mark.parametrize("qtype", WIDE, ids=[NAMES[t] for t in WIDE])
@pytest.mark.parametrize("N,K,kind", [(8192 + 4 * 37, 3584, "random"),
                                      (8192 + 16 * 9 + 5, 3072, "quantized"),
                                      (8192 + 16 * 5, 4096, "random"),
                                      (8192 + 7, 3328, "random")],
                         ids=["ragged_tile_K3584", "twelve_chunks", "sixteen_chunks", "thirteen_chunks"])
def test_gemv_wide_matrix_core_path(qtype, N, K, kind):
    """Wide Q8_0, Q4_0 and Q5_0 matrices (256-value super-chunks of 272, 144 and 176 bytes,
    whole 16-byte chunks) take the per-wave matrix-core kernel: a ragged last tile, idle waves
    (K = 3072), every wave busy (K = 4096), random block fields (any code, negative
    scales and minima), and an x with all-zero and tiny blocks and runs."""
    raw = weights(qtype, N, K, kind, 12)
    x = synth.activations(1, K, config_index=10, tensor_index=N % 73)[0]
    x[32:64] = 0.0
    x[112:128] *= 1e-30
    run_gemv(raw, qtype, x, N, K, what=f"{kind} wide")
    assert mq.last_kernel() == f"gemv_mfma<{NAMES[qtype]}>"


@pytest.mark.parametrize("qtype", WIDE, ids=[NAMES[t] for t in WIDE])
@pytest.mark.parametrize("N,K", [(16384 + 16 * 3 + 9, 3584), (37888 + 5, 3072)],
                         ids=["four_or_five_tiles", "nine_or_ten_tiles"])
def test_gemv_wide_many_tiles_per_workgroup(qtype, N, K):
    """The per-wave kernel with many 16-row tiles per workgroup: workgroups with 4, 5, 9 and
    10 tiles (ring loop groups of two with remainders of 0 and 1), checked on every row of
    the tiles of the first, second and last workgroups, the first and last 64 tiles and
    1000 random rows."""
    import torch
    G = torch.cuda.get_device_properties(device()).multi_processor_count
    T = (N + 15) // 16
    tiles = np.r_[0:64, T - 64:T, np.arange(0, T, G), np.arange(1, T, G), np.arange(G - 1, T, G)]
    rng = np.random.default_rng(N)
    rows = np.unique(np.r_[(tiles[:, None] * 16 + np.arange(16)).ravel(), rng.choice(N, 1000, replace=False)])
    rows = rows[rows < N]
    raw = weights(qtype, N, K, "random", 13)
    x = synth.activations(1, K, config_index=10, tensor_index=N % 71)[0]
    run_gemv(raw, qtype, x, N, K, rows=rows, what="wide, many tiles")
    assert mq.last_kernel() == f"gemv_mfma<{NAMES[qtype]}>"


def test_gemv_q8_0_wide_saturated_codes():
    """Wide Q8_0 runs reach |sum code * v| = 16 * 128 * 2^21 = 2^32 when every code of a
    16-value run is +-127 or -128 and x is constant just below a power of two in a block
    (the run's 21-bit digit form is then near its maximum): the run's three digit-plane
    sums must be combined without int32 wrap-around.  Rows: all +127, all -128, alternating
    runs of both, and random codes with -128 included; x blocks constant at 0.9, -0.75 and
    0.99999, plus N(0, 1) blocks."""
    N, K = 8192 + 64, 3584
    nb = K // 32
    rng = np.random.default_rng(77)
    codes = rng.integers(-128, 128, size=(N, nb, 32), dtype=np.int64)
    codes[0::4] = 127
    codes[1::4] = -128
    codes[2::4, :, :16] = 127
    codes[2::4, :, 16:] = -128
    d = np.full((N, nb), 0.0078125, dtype=np.float16)   # 2^-7, exact in f16
    d[3::4] = np.float16(-0.01)
    raw = np.zeros((N, nb, 34), dtype=np.uint8)
    raw[:, :, 0:2] = d[..., None].view(np.uint8).reshape(N, nb, 2)
    raw[:, :, 2:] = codes.astype(np.int8).view(np.uint8)
    x = synth.activations(1, K, config_index=10, tensor_index=41)[0]
    xb = x.reshape(nb, 32)
    xb[0::3] = np.float32(0.9)
    xb[1::3] = np.float32(-0.75)
    xb[2::6] = np.float32(0.99999)
    run_gemv(raw.reshape(-1), mq.Q8_0, x, N, K, what="saturated codes, wide")
    assert mq.last_kernel() == "gemv_mfma<q8_0>"
