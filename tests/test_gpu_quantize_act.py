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
    # the fp6 section (the activation operands of the Q4_K plane product) bit for bit
    got = mq.act_f6(Xq, M, K).cpu().numpy().reshape(-1)
    ref = oracle.act_f6_section(q, d, S)
    assert np.array_equal(got, ref), f"{what}: fp6 section differs at byte {int(np.argmax(got != ref))}"


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
