"""GPU parity of Q4_K's row-tiled layout (MQ_ROW_TILED) and of the long-row GEMV on it.

* The bytes mq_repack writes equal the oracle's row-tiled layout bit for bit,
  filler rows of a partial last group included.
* mq_gemv on it equals the GEMV on the GGUF payload bit for bit where that one runs the
  same long-row kernel with the same rows per workgroup (the 7B ffn_down shape, and the
  longest rows accepted), and is within 2e-4 of the oracle everywhere: one-row groups,
  a group with a filler row, more groups than CUs.
"""

import numpy as np
import pytest

import oracle
from block_quantized_matmul_mq_amd import mq, synth

from gpu_cases import check_normalized, device, row_norms, say, to_dev, weights

pytestmark = pytest.mark.gpu

T = mq.Q4_K | mq.ROW_TILED
KERNEL = "gemv_mfma_long<q4_K row-tiled>"


def tiled(raw, N, K, dev):
    import torch
    say(f"row-tiled repack q4_K N={N} K={K}")
    W = to_dev(raw.reshape(-1), dev)
    Wt = mq.repack(W, T, N, K)
    torch.cuda.synchronize()
    assert mq.last_kernel() == "repack"
    return W, Wt


@pytest.mark.parametrize("N,K", [(3, 17 * 256), (301, 17 * 256), (513, 18 * 256), (5000, 20 * 256)])
def test_repack_bytes_equal_the_oracle_layout(N, K):
    dev = device()
    raw = weights(mq.Q4_K, N, K, "random", 500 + N % 97)
    _, Wt = tiled(raw, N, K, dev)
    got = Wt.cpu().numpy()
    ref = oracle.q4_k_row_tiled(raw, N, K)
    assert got.size == mq.repack_bytes(T, N, K) == ref.size
    assert np.array_equal(got, ref), f"first difference at byte {np.argmax(got != ref)}"


@pytest.mark.parametrize("N,K,same_kernel", [(3584, 18944, True), (3584, 32768, True), (3, 17 * 256, False),
                                             (301, 17 * 256, False), (5000, 20 * 256, False)],
                         ids=["7b_ffn_down", "max_k", "one_row_groups", "filler_row", "313_groups"])
def test_gemv_on_row_tiled_weights(N, K, same_kernel):
    import torch
    dev = device()
    raw = synth.quantized_weight(mq.Q4_K, N, K, 1, 1) if N == 3584 else weights(mq.Q4_K, N, K, "quantized", N)
    W, Wt = tiled(raw, N, K, dev)
    xh = synth.activations(1, K, config_index=1, tensor_index=11)[0]
    x = to_dev(xh, dev)
    say(f"row-tiled gemv q4_K N={N} K={K}")
    yt = mq.gemv(Wt, T, x, N, K)
    torch.cuda.synchronize()
    assert mq.last_kernel() == KERNEL, mq.last_kernel()
    y = mq.gemv(W, mq.Q4_K, x, N, K)
    torch.cuda.synchronize()
    if same_kernel:
        assert mq.last_kernel() == "gemv_mfma_long<q4_K>", mq.last_kernel()
        a, b = yt.cpu().numpy(), y.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), \
            f"{np.count_nonzero(a.view(np.uint32) != b.view(np.uint32))} rows differ from the GGUF payload's"
    ref = oracle.gemv(raw, mq.Q4_K, xh, N, K)
    check_normalized(yt.cpu().numpy()[None, :], ref[None, :], row_norms(raw, mq.Q4_K, N, K),
                     np.array([np.linalg.norm(xh.astype(np.float64))]), f"row-tiled N={N} K={K}")


def test_wrong_length_and_the_prefill_are_refused():
    import torch
    dev = device()
    N, K = 301, 17 * 256
    raw = weights(mq.Q4_K, N, K, "random", 7)
    W, Wt = tiled(raw, N, K, dev)
    x = torch.zeros(K, device=dev)
    with pytest.raises(mq.MQError) as e:
        mq.gemv(W, T, x, N, K)                 # the GGUF payload is 144 x 17 bytes short of the layout
    assert e.value.code == -4
    Xq = mq.quantize_act(torch.zeros(40, K, device=dev))
    with pytest.raises(mq.MQError) as e:
        mq.gemm(Wt, T, Xq, 40, N, K)
    assert e.value.code == -3
