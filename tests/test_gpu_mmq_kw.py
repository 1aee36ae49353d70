"""GPU parity of the Q4_K product with one 32 x 32 output tile per workgroup and the
K range split over its four waves (mmq_kw<q4_K>), which mq_gemm takes for Q4_K on the
GGUF layout when the int8 kernel would have few 32-row tiles (a small N or M).

* Routing: the shapes below run this kernel and need no scratch.
* The exact int32 block dots it exports equal the oracle's bit for bit.
* Y is within 2e-4 of the oracle's f64 product (normalized per element), on every
  column of the 7B attn_k/attn_v prefill product (M = 512, 512 x 3584) and on K values
  that give every wave-range length from 0 to 8 steps of 128 values (loop groups of
  three plus remainders of 0, 1 and 2), with ragged row and column tiles.
"""

import numpy as np
import pytest

import oracle
from block_quantized_matmul_mq_amd import mq, synth

from gpu_cases import check_normalized, device, row_norms, say, to_dev, weights

pytestmark = pytest.mark.gpu

KERNEL = "mmq_kw<q4_K>"
Q4K = mq.Q4_K


def run(raw, X, N, K, blockdots, cols=None, what=""):
    import torch
    dev = device()
    M = X.shape[0]
    say(f"mmq_kw q4_K M={M} N={N} K={K} {what}")
    assert mq.gemm_scratch_bytes(Q4K, M, N, K) == 0
    W = to_dev(raw.reshape(-1), dev)
    Xq = mq.quantize_act(to_dev(X, dev))
    q, d, _ = oracle.quantize_act(X)
    if blockdots:
        D = mq.gemm_blockdots(W, Q4K, Xq, M, N, K)
        torch.cuda.synchronize()
        assert mq.last_kernel() == KERNEL, mq.last_kernel()
        ref = oracle.block_dots(raw, Q4K, q, N, K)
        got = D.cpu().numpy()
        assert np.array_equal(got, ref), f"{what}: block dots differ at {np.argwhere(got != ref)[:5]}"
    Y = mq.gemm(W, Q4K, Xq, M, N, K)
    torch.cuda.synchronize()
    assert mq.last_kernel() == KERNEL, mq.last_kernel()
    cols = np.arange(N) if cols is None else cols
    xh = (q.reshape(M, -1, 32).astype(np.float64) * d[..., None].astype(np.float64)).reshape(M, K)
    Y_ref = oracle.mmq(raw.reshape(N, -1)[cols], Q4K, q, d, len(cols), K)
    check_normalized(Y.cpu().numpy()[:, cols], Y_ref, row_norms(raw, Q4K, N, K, cols),
                     np.linalg.norm(xh, axis=1), f"M={M} {N}x{K} {what}")


@pytest.mark.parametrize("K", [256, 768, 1536, 2560, 3584, 4096],
                         ids=["ranges_0_1", "ranges_1_2", "ranges_3", "ranges_5", "ranges_7", "ranges_8"])
def test_wave_ranges_and_ragged_tiles(K):
    # M = 45: a second row tile of 13 rows; N = 300: a last column tile of 12 columns (at
    # K = 4096, N = 1700 and a last column tile of 4: with 300 columns the int8 kernel's
    # ranges would be short enough for it to be taken)
    M, N = 45, (1700 if K == 4096 else 300)
    raw = weights(Q4K, N, K, "random", 400 + K // 256)
    X = synth.activations(M, K, config_index=12, tensor_index=400 + K // 256)
    run(raw, X, N, K, blockdots=True, what=f"K={K}")


@pytest.mark.parametrize("M,N,K", [(9, 1, 256), (9, 33, 512), (32, 32, 1024), (33, 4096, 1024), (200, 2560, 2560)])
def test_edge_shapes(M, N, K):
    # one row above the multi-row GEMV's limit; a single column; exactly one tile; two
    # row tiles of which the second holds one row; and 560 tiles (more than one round)
    raw = weights(Q4K, N, K, "quantized", 420 + M)
    X = synth.activations(M, K, config_index=12, tensor_index=420 + M)
    rng = np.random.default_rng(M)
    cols = None if N <= 1024 else np.unique(np.r_[0:64, N - 64:N, rng.choice(N, 200, replace=False)])
    run(raw, X, N, K, blockdots=N <= 1024, cols=cols, what="edge")


def test_extreme_activations():
    M, N, K = 40, 96, 1536
    raw = weights(Q4K, N, K, "random", 430)
    X = synth.activations(M, K, config_index=14)
    X[0] = 0.0
    X[1, :64] = 0.0
    X[2] *= np.float32(1e-30)
    X[3] *= np.float32(1e30)
    X[4, ::7] = np.float32(50.0)
    X[5, :32] = np.float32(127.0) * np.sign(X[5, :32])
    run(raw, X, N, K, blockdots=True, what="extreme activations")


@pytest.mark.parametrize("tensor", [2, 3], ids=["attn_k", "attn_v"])
def test_7b_attn_kv_prefill_every_column(tensor):
    # the 7B attn_k / attn_v product at M = 512 (512 x 3584), in the launch configuration
    # the benchmark times, against the oracle on every output element
    M, N, K = 512, 512, 3584
    raw = synth.quantized_weight(Q4K, N, K, 3, tensor)
    X = synth.activations(M, K, 3)
    run(raw, X, N, K, blockdots=False, what="7B attn_k/v")


def test_long_k_few_tiles_stays_on_the_int8_kernel():
    # 24 tiles of 32 x 128 at K = 32768: the waves here would run 64 steps against the int8
    # kernel's ranges of 26, so that kernel (K cut across workgroups) is taken
    M, N, K = 20, 3000, 32768
    assert mq.gemm_scratch_bytes(Q4K, M, N, K) > 0
    import torch
    dev = device()
    say(f"routing q4_K M={M} N={N} K={K}")
    raw = weights(Q4K, N, K, "random", 440)
    X = synth.activations(M, K, config_index=12, tensor_index=440)
    Xq = mq.quantize_act(to_dev(X, dev))
    cols = np.r_[0:40, N - 40:N]
    Y = mq.gemm(to_dev(raw.reshape(-1), dev), Q4K, Xq, M, N, K)
    torch.cuda.synchronize()
    assert mq.last_kernel() == "mmq<q4_K>", mq.last_kernel()
    q, d, _ = oracle.quantize_act(X)
    xh = (q.reshape(M, -1, 32).astype(np.float64) * d[..., None].astype(np.float64)).reshape(M, K)
    Y_ref = oracle.mmq(raw.reshape(N, -1)[cols], Q4K, q, d, len(cols), K)
    check_normalized(Y.cpu().numpy()[:, cols], Y_ref, row_norms(raw, Q4K, N, K, cols),
                     np.linalg.norm(xh, axis=1), "long K, int8 kernel")
