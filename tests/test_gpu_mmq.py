"""GPU parity of mq_gemm (the int8 MMQ path) against the oracle.

* The exact int32 block dots the kernel forms (test export from the same
  kernel template) equal the oracle's block dots bit for bit.
* Y is within 2e-4 of the oracle's f64 product of deq(q8(X)) and deq(W),
  normalized per element by ||deq(W)[n]|| * ||x_hat[m]||.
"""

import numpy as np
import pytest

import oracle
from block_quantized_matmul_mq_amd import mq, synth

from gpu_cases import ALL_TYPES, BLOCK, NAMES, check_normalized, device, row_norms, say, to_dev, weights

pytestmark = pytest.mark.gpu

TYPES = ALL_TYPES


def quantized_plane(X, dev):
    import torch
    M, K = X.shape
    Xq = mq.quantize_act(to_dev(X, dev))
    torch.cuda.synchronize()
    return Xq


def x_hat_norms(X):
    q, d, _ = oracle.quantize_act(X)
    M, K = X.shape
    xh = (q.reshape(M, -1, 32).astype(np.float64) * d[..., None].astype(np.float64)).reshape(M, K)
    return np.linalg.norm(xh, axis=1), q, d


def check_blockdots(raw, qtype, X, N, K, what):
    import torch
    dev = device()
    M = X.shape[0]
    say(f"blockdots {NAMES[qtype]} M={M} N={N} K={K} {what}")
    Xq = quantized_plane(X, dev)
    D = mq.gemm_blockdots(to_dev(raw.reshape(-1), dev), qtype, Xq, M, N, K)
    torch.cuda.synchronize()
    assert mq.last_kernel().startswith(("mmq", "gemv_q8"))
    D = D.cpu().numpy()
    q, _, _ = oracle.quantize_act(X)
    ref = oracle.block_dots(raw, qtype, q, N, K)
    assert np.array_equal(D, ref), f"{what}: block dots differ at {np.argwhere(D != ref)[:5]}"


def check_gemm(raw, qtype, X, N, K, cols=None, what=""):
    import torch
    dev = device()
    M = X.shape[0]
    say(f"gemm {NAMES[qtype]} M={M} N={N} K={K} {what}")
    Xq = quantized_plane(X, dev)
    Y = mq.gemm(to_dev(raw.reshape(-1), dev), qtype, Xq, M, N, K)
    torch.cuda.synchronize()
    assert mq.last_kernel().startswith(("mmq", "gemv_q8"))
    Y = Y.cpu().numpy()
    cols = np.arange(N) if cols is None else cols
    xn, q, d = x_hat_norms(X)
    sub = raw.reshape(N, -1)[cols]
    Y_ref = oracle.mmq(sub, qtype, q, d, len(cols), K)
    wn = row_norms(raw, qtype, N, K, cols)
    return check_normalized(Y[:, cols], Y_ref, wn, xn, f"{NAMES[qtype]} M={M} {N}x{K} {what}")


def small_cases(qtype):
    b = BLOCK[qtype]
    return [(1, 1, b), (3, 33, 2 * b), (37, 130, 4 * b), (130, 300, 2 * b + 512), (129, 257, 1024)]


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
@pytest.mark.parametrize("kind", ["quantized", "random"])
def test_blockdots_bitwise_small_ragged(qtype, kind):
    for i, (M, N, K) in enumerate(small_cases(qtype)):
        raw = weights(qtype, N, K, kind, 20 + i)
        X = synth.activations(M, K, config_index=12, tensor_index=i)
        check_blockdots(raw, qtype, X, N, K, kind)


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
def test_split_k_uneven_ranges(qtype):
    # One output tile and a long K: the kernel splits K into many ranges of whole
    # 128-value steps (uneven lengths; for Q8_0 the last step is cut by K) and sums
    # the partials in a second launch.
    M, N, K = 40, 100, (4128 if BLOCK[qtype] == 32 else 8192)
    assert mq.gemm_scratch_bytes(qtype, M, N, K) >= 8 * M * N * 4, "shape must take the split-K path"
    raw = weights(qtype, N, K, "random", 70)
    X = synth.activations(M, K, config_index=12, tensor_index=30)
    check_blockdots(raw, qtype, X, N, K, "split-K")
    check_gemm(raw, qtype, X, N, K, what="split-K")


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
def test_small_m_multirow_gemv(qtype):
    # M <= 8 runs the multi-row GEMV over the quantized plane (rows padded to 1, 2, 4 or 8
    # in the kernel), ragged N and a K of several units; its block dots are exported by
    # the same kernel template.
    K = 2 * BLOCK[qtype] + 512
    for i, M in enumerate([1, 2, 3, 5, 8]):
        N = 300 + 7 * i
        raw = weights(qtype, N, K, "random", 110 + i)
        X = synth.activations(M, K, config_index=12, tensor_index=60 + i)
        check_blockdots(raw, qtype, X, N, K, f"M={M}")
        assert mq.last_kernel().startswith("gemv_q8")
        check_gemm(raw, qtype, X, N, K, what=f"M={M}")
        assert mq.last_kernel().startswith("gemv_q8")
        assert mq.gemm_scratch_bytes(qtype, M, N, K) == 0


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
def test_small_m_long_rows(qtype):
    # A long row still fits the multi-row GEMV's LDS at M = 4; at M = 8 and K = 32768 it
    # does not, and the product runs on the MMQ kernel with 32-row tiles.
    for M, K, N, path in [(4, 18944, 700, "gemv_q8"), (8, 32768, 260, "mmq")]:
        raw = weights(qtype, N, K, "random", 120 + M)
        X = synth.activations(M, K, config_index=12, tensor_index=70 + M)
        check_gemm(raw, qtype, X, N, K, what=f"M={M} K={K}")
        assert mq.last_kernel().startswith(path), mq.last_kernel()


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
def test_small_m_tiles_at_the_switch(qtype):
    # M <= 32 uses 32-row output tiles, M = 33 the 128-row ones; both with a ragged N.
    K = 2 * BLOCK[qtype] + 256
    for i, M in enumerate([32, 33]):
        N = 200
        raw = weights(qtype, N, K, "random", 90 + i)
        X = synth.activations(M, K, config_index=12, tensor_index=40 + i)
        check_blockdots(raw, qtype, X, N, K, f"M={M}")
        check_gemm(raw, qtype, X, N, K, what=f"M={M}")


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
def test_whole_tiles_plus_split_tail(qtype):
    # 520 output tiles: 512 computed whole, the last 8 cut into K ranges and summed by the
    # second launch; columns are sampled from both kinds of tile (the last 8 tiles are the
    # last 1024 columns).
    M, N, K = 100, 128 * 520, 512
    assert mq.gemm_scratch_bytes(qtype, M, N, K) == 2 * 8 * 128 * 128 * 4
    raw = weights(qtype, N, K, "quantized", 80)
    X = synth.activations(M, K, config_index=12, tensor_index=31)
    rng = np.random.default_rng(5)
    cols = np.sort(np.concatenate([rng.choice(N - 1024, 200, replace=False), np.arange(N - 1024, N)]))
    check_gemm(raw, qtype, X, N, K, cols=cols, what="whole + split tiles")


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
@pytest.mark.parametrize("kind", ["quantized", "random"])
def test_gemm_small_ragged(qtype, kind):
    for i, (M, N, K) in enumerate(small_cases(qtype)):
        raw = weights(qtype, N, K, kind, 40 + i)
        X = synth.activations(M, K, config_index=13, tensor_index=i)
        check_gemm(raw, qtype, X, N, K, what=kind)


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
def test_gemm_extreme_activations(qtype):
    M, N, K = 24, 96, 2 * BLOCK[qtype] + 256
    raw = weights(qtype, N, K, "random", 60)
    X = synth.activations(M, K, config_index=14)
    X[0] = 0.0
    X[1, :64] = 0.0
    X[2] *= np.float32(1e-30)
    X[3] *= np.float32(1e30)
    X[4, ::7] = np.float32(50.0)
    check_blockdots(raw, qtype, X, N, K, "extreme activations")
    check_gemm(raw, qtype, X, N, K, what="extreme activations")


def test_blockdots_config1_q8_0_m16():
    N, K = 4864, 896
    raw = synth.quantized_weight(mq.Q8_0, N, K, 0, 0)
    X = synth.activations(16, K, config_index=0)
    check_blockdots(raw, mq.Q8_0, X, N, K, "0.5B ffn_up M=16")
    check_gemm(raw, mq.Q8_0, X, N, K, what="0.5B ffn_up M=16")


@pytest.mark.parametrize("N,K,tensor", [(18944, 3584, 0), (3584, 3584, 1), (512, 3584, 2)],
                         ids=["ffn_up", "attn_q", "attn_kv"])
def test_gemm_config4_m512(N, K, tensor):
    raw = synth.quantized_weight(mq.Q4_K, N, K, 3, tensor)
    X = synth.activations(512, K, config_index=3)
    cols = None if N <= 4096 else np.random.default_rng(2).choice(N, 1024, replace=False)
    check_gemm(raw, mq.Q4_K, X, N, K, cols=cols, what="7B prefill M=512")


def test_blockdots_config4_sampled_tiles():
    # bit-exact block dots at the full ffn_up shape on a sub-block of rows/cols:
    # the export runs the whole grid; the comparison covers 3 x 2 tiles.
    N, K = 18944, 3584
    raw = synth.quantized_weight(mq.Q4_K, N, K, 3, 0)
    X = synth.activations(512, K, config_index=3)
    import torch
    dev = device()
    say("blockdots q4_K M=512 18944x3584 (sampled tiles)")
    Xq = quantized_plane(X, dev)
    D = mq.gemm_blockdots(to_dev(raw.reshape(-1), dev), mq.Q4_K, Xq, 512, N, K)
    torch.cuda.synchronize()
    q, _, _ = oracle.quantize_act(X)
    rows = np.r_[0:128, 384:512]
    cols = np.r_[0:256, N - 128:N]
    ref = oracle.block_dots(raw.reshape(N, -1)[cols], mq.Q4_K, q[rows], len(cols), K)
    got = D[torch.from_numpy(rows).to(dev)][:, torch.from_numpy(cols).to(dev)].cpu().numpy()
    assert np.array_equal(got, ref)


def test_gemm_config3_m8_head_sampled():
    N, K = 152064, 3584
    raw = synth.quantized_weight(mq.Q6_K, N, K, 2, 0)
    X = synth.activations(8, K, config_index=2, tensor_index=8)
    cols = np.unique(np.concatenate([np.random.default_rng(3).choice(N, 2000, replace=False),
                                     np.arange(N - 40, N)]))
    check_gemm(raw, mq.Q6_K, X, N, K, cols=cols, what="head M=8 (sampled cols)")


@pytest.mark.parametrize("qtype,N,K,tensor", [(mq.Q4_K, 5120, 5120, 0), (mq.Q4_K, 1024, 5120, 1),
                                              (mq.Q4_K, 13824, 5120, 2), (mq.Q6_K, 5120, 13824, 3)],
                         ids=["attn_q", "attn_k", "ffn_up", "ffn_down"])
def test_gemm_config5_m2048_sampled(qtype, N, K, tensor):
    raw = synth.quantized_weight(qtype, N, K, 4, tensor)
    X = synth.activations(2048, K, config_index=4, tensor_index=10 + (K == 13824))
    cols = np.random.default_rng(4).choice(N, 384, replace=False)
    check_gemm(raw, qtype, X, N, K, cols=cols, what="14B prefill M=2048 (sampled cols)")


@pytest.mark.parametrize("N,K,kind", [(8192 + 4 * 37, 3584, "random"), (8192 + 16 * 9, 3072, "quantized"),
                                      (8192 + 16 * 5, 4096, "random"), (8192 + 8 * 11, 3328, "random")],
                         ids=["ragged_tile_K3584", "twelve_super_blocks", "sixteen_super_blocks", "odd_row_alignment"])
def test_small_m_q6_k_matrix_core_path(N, K, kind):
    """Wide Q6_K at M <= 8 takes the whole-tile matrix-core kernel over the q8 rows (one
    group of four rows for M <= 4, two above): bitwise block dots (the dot of code - 32
    with the q8 codes per 16-value group) and f32 parity, for M = 1, 3, 4, 5, 8, with a
    ragged last tile, idle waves (K = 3072) and every wave busy (K = 4096)."""
    raw = weights(mq.Q6_K, N, K, kind, 130)
    for i, M in enumerate([1, 3, 4, 5, 8]):
        X = synth.activations(M, K, config_index=12, tensor_index=80 + i)
        X[:, 32:64] = 0.0
        check_blockdots(raw, mq.Q6_K, X, N, K, f"M={M} {kind}")
        assert mq.last_kernel() == "gemv_q8_mfma<q6_K>", mq.last_kernel()
        check_gemm(raw, mq.Q6_K, X, N, K, what=f"M={M} {kind}")
        assert mq.last_kernel() == "gemv_q8_mfma<q6_K>", mq.last_kernel()
