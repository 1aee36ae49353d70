"""GPU parity of mq_quantize_act against the oracle: bit-exact codes, scales and sums."""

import numpy as np
import pytest

import oracle
from block_quantized_matmul_mq_amd import mq, synth

from gpu_cases import device, say, to_dev

pytestmark = pytest.mark.gpu


def run_and_compare(X, what):
    import torch
    dev = device()
    M, K = X.shape
    say(f"quantize_act {what} M={M} K={K}")
    Xq = mq.quantize_act(to_dev(X, dev))
    torch.cuda.synchronize()
    assert mq.last_kernel() == "quantize_act"
    codes, scales, sums = (t.cpu().numpy() for t in mq.split_act(Xq, M, K))
    q, d, S = oracle.quantize_act(X)
    assert np.array_equal(codes, q), f"{what}: codes differ at {np.argwhere(codes != q)[:5]}"
    assert np.array_equal(scales.view(np.uint32), d.view(np.uint32)), f"{what}: scales differ"
    assert np.array_equal(sums, S), f"{what}: sums differ"
    # the fp8 digit records re-encode the codes exactly: h and l bytes decoded as e4m3
    T = (K + 63) // 64
    rec = mq.act_digits(Xq, M, K).cpu().numpy().reshape(M, 2 * T, 2, 32)
    if K % 64:   # the last step's second block does not exist: all zero
        assert not rec[:, -1].any(), f"{what}: padding digits"
        rec = rec[:, :-1]
    hv = e4m3_values(rec[:, :, 0, :]) * 2.0 ** 9
    lv = e4m3_values(rec[:, :, 1, :]) * 2.0 ** 9
    assert np.all(np.abs(lv) <= 15) and np.all(hv == 16 * np.round(hv / 16)), f"{what}: digit ranges"
    assert np.all(np.abs(hv) <= 112), f"{what}: h digit range"
    decoded = (hv + lv).reshape(M, K)
    assert np.array_equal(decoded, q.astype(np.float64)), f"{what}: digit records differ from the codes"
    # both digits carry the code's sign (the l byte of a code with |q| % 16 == 0 may be +-0)
    assert np.all(np.sign(hv.reshape(M, K)) * np.sign(q) >= 0), f"{what}: digit signs"
    # step scale records: (scale, scale, sum, sum) of blocks 2t and 2t + 1, zero padded
    ss, sm = (t.cpu().numpy() for t in mq.act_step_scales(Xq, M, K))
    pad = 2 * T - K // 32
    dpad = np.concatenate([d, np.zeros((M, pad), np.float32)], axis=1).reshape(M, T, 2)
    spad = np.concatenate([S, np.zeros((M, pad), np.int32)], axis=1).reshape(M, T, 2)
    assert np.array_equal(ss.transpose(1, 0, 2).view(np.uint32), dpad.view(np.uint32)), f"{what}: step scales"
    assert np.array_equal(sm.transpose(1, 0, 2), spad), f"{what}: step sums"


def e4m3_values(b):
    """OCP e4m3 bytes -> float64 (no NaN bytes are expected here)."""
    b = b.astype(np.int64)
    assert not np.any((b & 0x7F) == 0x7F), "NaN byte"
    s = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (8 + m) * np.exp2(e - 10.0))
    return s * mag


@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (7, 4128), (5, 4160), (16, 896), (8, 3584), (512, 3584),
                                 (2048, 5120)])
def test_quantize_act_bitwise_normal(M, K):
    X = synth.activations(M, K, config_index=3, tensor_index=M)
    run_and_compare(X, "normal")


def test_quantize_act_bitwise_2048x13824():
    X = synth.activations(2048, 13824, config_index=4, tensor_index=7)
    run_and_compare(X, "14B ffn_down input")


def test_quantize_act_special_values():
    rng = np.random.default_rng(5)
    X = synth.normal_f32(rng, (12, 256))
    X[0] = 0.0                                            # zero blocks
    X[1, :32] = np.float32(3e38) * np.sign(X[1, :32])     # near f32 max
    X[2, :32] = np.float32(1e-40)                         # subnormal amax
    X[2, 32:64] *= np.float32(1e-39)                      # subnormal mixtures
    X[3, :32] = np.float32(0.5) * np.arange(-16, 16, dtype=np.float32)  # exact ties when amax->127
    X[3, 0] = np.float32(127.0)
    X[4, :] = -np.abs(X[4, :])                            # all negative
    X[5, ::32] = np.float32(1e6)                          # one outlier per block
    X[6, :32] = np.float32(889.0)                         # scale exactly 7
    X[6, 1:8] = np.float32([45.5, 87.5, 101.5, -45.5, 3.5, 10.5, -87.5])
    X[7] = -X[8]
    run_and_compare(X, "special")


def test_quantize_act_heavy_tails():
    X = synth.activations(64, 3584, config_index=3, tensor_index=77)
    rng = np.random.default_rng(9)
    idx = rng.integers(0, X.size, 200)
    X.reshape(-1)[idx] = rng.choice([-50.0, 50.0], 200).astype(np.float32)
    run_and_compare(X, "outliers")
