"""GPU parity of the Q4_0 / Q4_1 / Q5_0 / Q5_1 / Q5_K products at model shapes,
and of the concatenated gate/up weight (one 2N-row product).

The type whitelist of "minfer CUDA Backend Design", 4.3 Eligibility names these
types; the small and ragged cases of every type run in test_gpu_gemv.py and
test_gpu_mmq.py.  Here: the 32-value types on the Qwen2.5-0.5B ffn_up shape
(4864 x 896) at M = 1 (f32 GEMV), 16 (MMQ, bitwise block dots) and 8 (the
multi-row GEMV); Q5_K on the Qwen2.5-7B FFN shapes at M = 1 and M = 512.

The fused gate/up weight: the loader registers blk.{i}.ffn_gu, the gate and up
rows concatenated, and multiplies it as one matmul ("minfer CUDA Backend
Design", 4.6 Model wiring).  Rows are independent, so the product
of the concatenation must agree with the two products, each within the
tolerance of the oracle.
"""

import numpy as np
import pytest

import oracle
from block_quantized_matmul_mq_amd import mq, synth

from gpu_cases import NAMES, check_normalized, device, row_norms, say, to_dev

pytestmark = pytest.mark.gpu

LEGACY = [mq.Q4_0, mq.Q4_1, mq.Q5_0, mq.Q5_1]


def _x_hat_norms(X):
    q, d, _ = oracle.quantize_act(X)
    M, K = X.shape
    xh = (q.reshape(M, -1, 32).astype(np.float64) * d[..., None].astype(np.float64)).reshape(M, K)
    return np.linalg.norm(xh, axis=1), q, d


def _gemv_check(raw, qtype, x, N, K, what, rows=None):
    import torch
    dev = device()
    say(f"gemv {NAMES[qtype]} N={N} K={K} {what}")
    y = mq.gemv(to_dev(raw.reshape(-1), dev), qtype, to_dev(x, dev), N, K)
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    rows = np.arange(N) if rows is None else rows
    y_ref = oracle.gemv(raw.reshape(N, -1)[rows], qtype, x, len(rows), K)
    wn = row_norms(raw, qtype, N, K, rows)
    xn = np.array([np.linalg.norm(x.astype(np.float64))])
    check_normalized(y[rows][None, :], y_ref[None, :], wn, xn, f"{NAMES[qtype]} {N}x{K} {what}")
    return y


def _gemm_check(raw, qtype, X, N, K, what, cols=None, blockdots=False):
    import torch
    dev = device()
    M = X.shape[0]
    say(f"gemm {NAMES[qtype]} M={M} N={N} K={K} {what}")
    W = to_dev(raw.reshape(-1), dev)
    Xq = mq.quantize_act(to_dev(X, dev))
    Y = mq.gemm(W, qtype, Xq, M, N, K)
    torch.cuda.synchronize()
    kernel = mq.last_kernel()
    Y = Y.cpu().numpy()
    xn, q, d = _x_hat_norms(X)
    cols = np.arange(N) if cols is None else cols
    sub = raw.reshape(N, -1)[cols]
    Y_ref = oracle.mmq(sub, qtype, q, d, len(cols), K)
    check_normalized(Y[:, cols], Y_ref, row_norms(raw, qtype, N, K, cols), xn, f"{NAMES[qtype]} M={M} {what}")
    if blockdots:
        D = mq.gemm_blockdots(W, qtype, Xq, M, N, K)
        torch.cuda.synchronize()
        assert mq.last_kernel() == kernel
        assert np.array_equal(D.cpu().numpy(), oracle.block_dots(raw, qtype, q, N, K)), f"{what}: block dots"
    return Y, kernel


@pytest.mark.parametrize("qtype", LEGACY, ids=[NAMES[t] for t in LEGACY])
def test_32_value_types_on_the_0_5b_ffn_up_shape(qtype):
    N, K = 4864, 896
    raw = synth.quantized_weight(qtype, N, K, 0, 20 + qtype)
    X = synth.activations(16, K, config_index=0, tensor_index=20 + qtype)
    _gemv_check(raw, qtype, X[0], N, K, "0.5B ffn_up")
    _, kern = _gemm_check(raw, qtype, X, N, K, "0.5B ffn_up M=16", blockdots=True)
    assert kern.startswith("mmq"), kern
    _, kern = _gemm_check(raw, qtype, X[:8], N, K, "0.5B ffn_up M=8", blockdots=True)
    assert kern.startswith("gemv_q8"), kern


@pytest.mark.parametrize("N,K,tensor", [(18944, 3584, 0), (3584, 18944, 1)], ids=["ffn_up", "ffn_down"])
def test_q5_k_on_the_7b_ffn_shapes(N, K, tensor):
    raw = synth.quantized_weight(mq.Q5_K, N, K, 1, 40 + tensor)
    x = synth.activations(1, K, config_index=1, tensor_index=40 + tensor)[0]
    _gemv_check(raw, mq.Q5_K, x, N, K, "7B FFN")


def test_q5_k_prefill_m512_sampled():
    N, K = 18944, 3584
    raw = synth.quantized_weight(mq.Q5_K, N, K, 3, 40)
    X = synth.activations(512, K, config_index=3, tensor_index=40)
    rng = np.random.default_rng(3)
    cols = np.sort(np.concatenate([rng.choice(N - 1024, 300, replace=False), np.arange(N - 128, N)]))
    _, kern = _gemm_check(raw, mq.Q5_K, X, N, K, "7B ffn_up M=512", cols=cols)
    assert kern.startswith("mmq"), kern


@pytest.mark.parametrize("qtype", [mq.Q4_K, mq.Q5_K, mq.Q4_0], ids=["q4_K", "q5_K", "q4_0"])
def test_concatenated_gate_up_matches_the_two_products(qtype):
    # ffn_gate and ffn_up (N rows each) as one 2N-row weight: one launch, one pass over x / Xq
    import torch
    dev = device()
    N, K = 2368, 3584          # an 8-way share of the 7B FFN width, so the test stays small
    gate = synth.quantized_weight(qtype, N, K, 5, 1)
    up = synth.quantized_weight(qtype, N, K, 5, 2)
    gu = np.concatenate([gate.reshape(N, -1), up.reshape(N, -1)], axis=0)
    for M in (1, 8, 64):
        X = synth.activations(M, K, config_index=5, tensor_index=M)
        if M == 1:
            y = _gemv_check(gu, qtype, X[0], 2 * N, K, "gate|up")
            yg = _gemv_check(gate, qtype, X[0], N, K, "gate")
            yu = _gemv_check(up, qtype, X[0], N, K, "up")
            sep = np.concatenate([yg, yu])[None, :]
            y = y[None, :]
            xn = np.array([np.linalg.norm(X[0].astype(np.float64))])
        else:
            y, _ = _gemm_check(gu, qtype, X, 2 * N, K, "gate|up")
            yg, _ = _gemm_check(gate, qtype, X, N, K, "gate")
            yu, _ = _gemm_check(up, qtype, X, N, K, "up")
            sep = np.concatenate([yg, yu], axis=1)
            xn = _x_hat_norms(X)[0]
        wn = row_norms(gu, qtype, 2 * N, K)
        diff = np.abs(y.astype(np.float64) - sep.astype(np.float64)) / np.outer(xn, wn)
        say(f"  M={M}: fused vs separate max normalized difference {diff.max():.3e}")
        assert diff.max() <= 4e-4
    torch.cuda.synchronize()
