"""The MQ_ERR_LAUNCH path of every launching call: with mq_debug_refuse_launches the
next calls take the path of a launch the runtime refused (no kernel runs).  Each call
returns MQ_ERR_LAUNCH with a message naming the call, the kernel and the runtime error;
the binding raises MQError with that code; the next call launches again and gives the
bits of a call made before the refusals."""

import numpy as np
import pytest

from block_quantized_matmul_mq_amd import mq, synth

from gpu_cases import device, say, to_dev, weights

pytestmark = pytest.mark.gpu


def refused(fn, what):
    lib = mq.load()
    assert lib.mq_debug_refuse_launches(1) == 0
    with pytest.raises(mq.MQError) as e:
        fn()
    assert e.value.code == -7, e.value
    msg = mq.last_error()
    assert what in msg and "refused" in msg and "hipErrorLaunchFailure" in msg, msg


def test_every_launching_call_reports_a_refused_launch():
    import torch
    dev = device()
    mq.init(0)
    lib = mq.load()
    assert lib.mq_debug_refuse_launches(-1) == -1
    M, N, K = 40, 300, 512
    raw = weights(mq.Q4_K, N, K, "random", 400)
    W = to_dev(raw.reshape(-1), dev)
    X = to_dev(synth.activations(M, K, config_index=12, tensor_index=400), dev)
    x = X[0].contiguous()
    say("refused launches: quantize_act, gemv, gemm (int8), repack, gemm (fp6 plane), block dots, row-tiled")
    refused(lambda: mq.quantize_act(X), "mq_quantize_act: launch of quantize_act")
    Xq = mq.quantize_act(X)
    refused(lambda: mq.gemv(W, mq.Q4_K, x, N, K), "mq_gemv: launch of gemv")
    y = mq.gemv(W, mq.Q4_K, x, N, K)
    refused(lambda: mq.gemm(W, mq.Q4_K, Xq, M, N, K), "mq_gemm: launch of mmq")
    Y = mq.gemm(W, mq.Q4_K, Xq, M, N, K)
    refused(lambda: mq.repack(W, mq.Q4_K, N, K), "mq_repack: launch of repack")
    Wp = mq.repack(W, mq.Q4_K, N, K)
    plane = mq.Q4_K | mq.REPACKED
    refused(lambda: mq.gemm(Wp, plane, Xq, M, N, K), "mq_gemm: launch of mmq_f6<q4_K plane>")
    Yp = mq.gemm(Wp, plane, Xq, M, N, K)
    refused(lambda: mq.gemm_blockdots(W, mq.Q4_K, Xq, M, N, K), "mq_debug_gemm_blockdots: launch of mmq")
    # Q4_K's row-tiled layout and the long-row GEMV on it (rows of more than 16 super-blocks)
    Kt = 17 * 256
    Wl = to_dev(weights(mq.Q4_K, N, Kt, "random", 401).reshape(-1), dev)
    xt = to_dev(synth.activations(1, Kt, config_index=12, tensor_index=401)[0], dev)
    refused(lambda: mq.repack(Wl, mq.Q4_K | mq.ROW_TILED, N, Kt), "mq_repack: launch of repack")
    Wt = mq.repack(Wl, mq.Q4_K | mq.ROW_TILED, N, Kt)
    refused(lambda: mq.gemv(Wt, mq.Q4_K | mq.ROW_TILED, xt, N, Kt),
            "mq_gemv: launch of gemv_mfma_long<q4_K row-tiled>")
    yt = mq.gemv(Wt, mq.Q4_K | mq.ROW_TILED, xt, N, Kt)
    # two refusals in a row, then the calls launch again
    assert lib.mq_debug_refuse_launches(2) == 0
    for _ in range(2):
        with pytest.raises(mq.MQError):
            mq.gemv(W, mq.Q4_K, x, N, K)
    y2 = mq.gemv(W, mq.Q4_K, x, N, K)
    Y2 = mq.gemm(W, mq.Q4_K, Xq, M, N, K)
    Yp2 = mq.gemm(Wp, plane, Xq, M, N, K)
    yt2 = mq.gemv(Wt, mq.Q4_K | mq.ROW_TILED, xt, N, Kt)
    torch.cuda.synchronize()
    for a, b in ((y, y2), (Y, Y2), (Yp, Yp2), (yt, yt2)):
        a, b = a.cpu().numpy(), b.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
