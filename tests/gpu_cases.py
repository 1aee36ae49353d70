"""Shared helpers for the GPU parity tests: device setup, seeded inputs, and the
normalized-error check.

Tolerance: |Y - Y_ref| <= 2e-4 * ||deq(W)[n]|| * ||x_hat[m]|| per output element
(x_hat = x for the GEMV, deq(q8(x)) for the MMQ); a zero-norm row needs Y == 0.
Integer outputs (activation codes, block dots) must match exactly.
"""

import sys

import numpy as np

import oracle
from block_quantized_matmul_mq_amd import mq, synth

TOL = 2e-4

BLOCK = {mq.Q8_0: 32, mq.Q4_K: 256, mq.Q6_K: 256,
         mq.Q4_0: 32, mq.Q4_1: 32, mq.Q5_0: 32, mq.Q5_1: 32, mq.Q5_K: 256}
NAMES = {mq.Q8_0: "q8_0", mq.Q4_K: "q4_K", mq.Q6_K: "q6_K",
         mq.Q4_0: "q4_0", mq.Q4_1: "q4_1", mq.Q5_0: "q5_0", mq.Q5_1: "q5_1", mq.Q5_K: "q5_K"}
# every served weight type: the three of the measured workloads first, then the other
# types of the eligibility list
ALL_TYPES = [mq.Q8_0, mq.Q4_K, mq.Q6_K, mq.Q4_0, mq.Q4_1, mq.Q5_0, mq.Q5_1, mq.Q5_K]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def device():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a HIP device")
    mq.init(0)
    return torch.device("cuda:0")


def to_dev(arr, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)


def weights(qtype, N, K, kind, seed):
    if kind == "quantized":
        return synth.quantized_weight(qtype, N, K, 90, seed)
    rng = np.random.default_rng(1000 + seed)
    return synth.random_blocks(qtype, N, K, rng)


def row_norms(raw, qtype, N, K, rows=None):
    rows = np.arange(N) if rows is None else rows
    w = oracle.decode(raw.reshape(N, -1)[rows], qtype, len(rows), K)
    return np.linalg.norm(w, axis=1)


def check_normalized(y, y_ref, w_norm, x_norm, what):
    """y, y_ref: [M, n]; w_norm: [n]; x_norm: [M]."""
    y = np.asarray(y, dtype=np.float64)
    bound = TOL * np.outer(x_norm, w_norm)
    err = np.abs(y - y_ref)
    zero = bound == 0
    assert np.all(y[zero] == 0), f"{what}: nonzero output for a zero-norm row"
    ratio = np.where(zero, 0.0, err / np.where(zero, 1.0, bound))
    worst = float(ratio.max()) if ratio.size else 0.0
    say(f"  {what}: max normalized error = {worst * TOL:.3e} (bound {TOL:.0e})")
    assert worst <= 1.0, f"{what}: normalized error {worst * TOL:.3e} > {TOL}"
    return worst * TOL
