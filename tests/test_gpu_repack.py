"""GPU parity of mq_repack (the one-time device-layout transform) and of the products
on the repacked layout.

* The repacked bytes equal the oracle's repacked layout bit for bit.
* mq_gemv / mq_gemm / the block-dot export on type | MQ_REPACKED give exactly the
  same outputs as on the GGUF payload (the same kernels, only the block addresses
  differ), and the GEMV on the repacked head stays within 2e-4 of the oracle.
"""

import numpy as np
import pytest

import oracle
from block_quantized_matmul_mq_amd import mq, synth

from gpu_cases import NAMES, check_normalized, device, row_norms, say, to_dev, weights

pytestmark = pytest.mark.gpu

TYPES = [mq.Q8_0, mq.Q6_K]


def repacked(raw, qtype, N, K, dev):
    import torch
    say(f"repack {NAMES[qtype]} N={N} K={K}")
    W = to_dev(raw.reshape(-1), dev)
    Wr = mq.repack(W, qtype, N, K)
    torch.cuda.synchronize()
    assert mq.last_kernel() == "repack"
    return W, Wr


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
@pytest.mark.parametrize("N,K", [(1, 256), (37, 512), (300, 2048 + 256)])
def test_repack_bytes_equal_the_oracle_layout(qtype, N, K):
    dev = device()
    raw = weights(qtype, N, K, "random", N)
    _, Wr = repacked(raw, qtype, N, K, dev)
    got = Wr.cpu().numpy()
    ref = oracle.repack(raw, qtype, N, K)
    assert got.size == mq.repack_bytes(qtype, N, K) == ref.size
    assert np.array_equal(got, ref), f"first difference at byte {np.argmax(got != ref)}"


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
@pytest.mark.parametrize("N,K", [(130, 512), (4864, 896 + 128), (1029, 3584)])
def test_gemv_on_repacked_weights_is_identical(qtype, N, K):
    import torch
    dev = device()
    if K % (32 if qtype == mq.Q8_0 else 256):
        K -= K % 256
    raw = weights(qtype, N, K, "quantized", 3)
    W, Wr = repacked(raw, qtype, N, K, dev)
    x = to_dev(synth.activations(1, K, config_index=10, tensor_index=5)[0], dev)
    y = mq.gemv(W, qtype, x, N, K)
    yr = mq.gemv(Wr, qtype | mq.REPACKED, x, N, K)
    torch.cuda.synchronize()
    assert "repacked" in mq.last_kernel()
    assert torch.equal(y, yr), f"max diff {float((y - yr).abs().max())}"


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
@pytest.mark.parametrize("M,N,K", [(3, 130, 512), (40, 300, 1024), (130, 257, 2048)])
def test_gemm_and_blockdots_on_repacked_weights_are_identical(qtype, M, N, K):
    import torch
    dev = device()
    raw = weights(qtype, N, K, "random", 4)
    W, Wr = repacked(raw, qtype, N, K, dev)
    X = synth.activations(M, K, config_index=10, tensor_index=6)
    Xq = mq.quantize_act(to_dev(X, dev))
    Y = mq.gemm(W, qtype, Xq, M, N, K)
    Yr = mq.gemm(Wr, qtype | mq.REPACKED, Xq, M, N, K)
    D = mq.gemm_blockdots(W, qtype, Xq, M, N, K)
    Dr = mq.gemm_blockdots(Wr, qtype | mq.REPACKED, Xq, M, N, K)
    torch.cuda.synchronize()
    assert "repacked" in mq.last_kernel()
    assert torch.equal(D, Dr)
    assert torch.equal(Y, Yr), f"max diff {float((Y - Yr).abs().max())}"
    q, _, _ = oracle.quantize_act(X)
    assert np.array_equal(Dr.cpu().numpy(), oracle.block_dots(raw, qtype, q, N, K))


def test_gemv_repacked_q6_k_head_sampled():
    import torch
    dev = device()
    N, K = 152064, 3584
    raw = synth.quantized_weight(mq.Q6_K, N, K, 2, 0)
    W, Wr = repacked(raw, mq.Q6_K, N, K, dev)
    del W
    x = synth.activations(1, K, config_index=2)[0]
    y = mq.gemv(Wr, mq.Q6_K | mq.REPACKED, to_dev(x, dev), N, K)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.integers(0, N, 2000), np.arange(32), np.arange(N - 32, N)]))
    y_ref = oracle.gemv(raw.reshape(N, -1)[rows], mq.Q6_K, x, len(rows), K)
    xn = np.array([np.linalg.norm(x.astype(np.float64))])
    check_normalized(y[rows][None, :], y_ref[None, :], row_norms(raw, mq.Q6_K, N, K, rows), xn,
                     "repacked q6_K head (sampled rows)")
