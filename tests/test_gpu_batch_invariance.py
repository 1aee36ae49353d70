"""Batch invariance of mq_gemm on the small-M path.

For M <= 8, mq_gemm runs one multi-row GEMV whose per-output arithmetic (exact
int32 block dots, the same f32 scaling per unit and row, a sum over the row's
units in unit order) does not depend on how many rows share the launch.  So
row m of a product over M <= 8 rows must equal, bit for bit, the product of
that row alone (M = 1).  This mirrors the reference engine's rule that
multi-token products of up to 8 tokens are bitwise equal to the single-token
ones ("minfer Architecture Execution Plan", the multi-token decode rows).

At M = 9 the product moves to the MMQ tiles, whose accumulation order differs:
there the rows agree with the M = 1 results only to the product tolerance
(both are within 2e-4 of the oracle, so they differ by at most twice that),
which is the documented tolerance class of the switch.
"""

import numpy as np
import pytest

import oracle
from block_quantized_matmul_mq_amd import mq, synth

from gpu_cases import NAMES, TOL, check_normalized, device, row_norms, say, to_dev, weights

pytestmark = pytest.mark.gpu

TYPES = [mq.Q8_0, mq.Q4_K, mq.Q6_K]


def _gemm(W, qtype, X, N, K):
    import torch
    Xq = mq.quantize_act(to_dev(X, device()))
    Y = mq.gemm(W, qtype, Xq, X.shape[0], N, K)
    torch.cuda.synchronize()
    return Y.cpu().numpy(), mq.last_kernel()


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
def test_rows_of_small_m_equal_single_row_bitwise(qtype):
    dev = device()
    N, K = 300, 2048
    raw = weights(qtype, N, K, "quantized", 61)
    W = to_dev(raw.reshape(-1), dev)
    X = synth.activations(8, K, config_index=14, tensor_index=qtype)
    singles = []
    for m in range(8):
        y, kern = _gemm(W, qtype, X[m:m + 1], N, K)
        assert kern.startswith("gemv_q8"), kern
        singles.append(y[0])
    for M in (2, 3, 5, 8):
        say(f"batch invariance {NAMES[qtype]} M={M} N={N} K={K}")
        Y, kern = _gemm(W, qtype, X[:M], N, K)
        assert kern.startswith("gemv_q8"), kern
        for m in range(M):
            assert np.array_equal(Y[m].view(np.uint32), singles[m].view(np.uint32)), \
                f"M={M} row {m} differs from its M=1 product at {np.flatnonzero(Y[m] != singles[m])[:5]}"


def test_vocab_head_m8_rows_equal_single_rows_bitwise():
    # the speculative-verify batch of the vocab head: M = 8 against 8 single-row products
    dev = device()
    N, K = 152064, 3584
    raw = synth.quantized_weight(mq.Q6_K, N, K, 2, 0)
    W = to_dev(raw.reshape(-1), dev)
    X = synth.activations(8, K, 2, tensor_index=5)
    say(f"batch invariance q6_K head M=8 N={N} K={K}")
    Y, kern = _gemm(W, mq.Q6_K, X, N, K)
    assert kern.startswith("gemv_q8"), kern
    for m in range(8):
        y, _ = _gemm(W, mq.Q6_K, X[m:m + 1], N, K)
        assert np.array_equal(Y[m].view(np.uint32), y[0].view(np.uint32)), f"head row {m} differs"


@pytest.mark.parametrize("qtype", TYPES, ids=[NAMES[t] for t in TYPES])
def test_switch_to_mmq_is_a_tolerance_class(qtype):
    # M = 9 runs the MMQ tiles: each row is within the product tolerance of the oracle, and
    # so within twice that of the M = 1 product of the same row.
    dev = device()
    N, K = 300, 2048
    raw = weights(qtype, N, K, "quantized", 62)
    W = to_dev(raw.reshape(-1), dev)
    X = synth.activations(9, K, config_index=14, tensor_index=20 + qtype)
    say(f"switch M=9 {NAMES[qtype]} N={N} K={K}")
    Y9, kern = _gemm(W, qtype, X, N, K)
    assert kern.startswith("mmq"), kern
    q, d, _ = oracle.quantize_act(X)
    xh = (q.reshape(9, -1, 32).astype(np.float64) * d[..., None].astype(np.float64)).reshape(9, K)
    xn = np.linalg.norm(xh, axis=1)
    wn = row_norms(raw, qtype, N, K)
    Y_ref = oracle.mmq(raw, qtype, q, d, N, K)
    check_normalized(Y9, Y_ref, wn, xn, f"{NAMES[qtype]} M=9 (MMQ tiles)")
    worst = 0.0
    for m in range(9):
        y1, kern1 = _gemm(W, qtype, X[m:m + 1], N, K)
        assert kern1.startswith("gemv_q8"), kern1
        bound = xn[m] * wn
        diff = np.abs(Y9[m].astype(np.float64) - y1[0].astype(np.float64))
        ratio = np.where(bound > 0, diff / np.where(bound > 0, bound, 1.0), 0.0)
        worst = max(worst, float(ratio.max()))
    say(f"  M=9 rows vs their M=1 products: max normalized difference {worst:.3e}")
    assert worst <= 2 * TOL
