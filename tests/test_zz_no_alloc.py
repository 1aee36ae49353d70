"""mq_gemm_noalloc (the product with the library's per-device scratch array) gives
the same bits as mq_gemm with a caller-allocated, zeroed scratch buffer, over calls
in a row that reuse the array: K-split int8 products (GGUF payload, 128- and 32-row
tiles) and K-split fp6 products (Q4_K's MMQ plane) whose partial tiles overwrite each
other's and which cut different numbers of tiles (the shared counters must still read
zero), and products that cut none."""

import numpy as np
import pytest

from block_quantized_matmul_mq_amd import mq, synth

from gpu_cases import device, say, to_dev, weights

pytestmark = pytest.mark.gpu

CASES = [
    # (M, N, K, kernel, partial-tile bytes the plan cuts); the plane kernel reads Q4_K's MMQ
    # plane (mq_repack); both kernels count cut tiles in the same counters
    (512, 18944, 3584, "mmq<q4_K>", 80 * 3 * 128 * 128 * 4),        # ffn_up: 80 tiles cut into 3
    (512, 18944, 3584, "mmq_f6<q4_K plane>", 80 * 3 * 128 * 128 * 4),   # the plane: 80 into 3
    (40, 100, 8192, "mmq_f6<q4_K plane>", 1 * 32 * 128 * 128 * 4),      # one tile into 32
    (40, 100, 8192, "mmq<q4_K>", 2 * 32 * 32 * 128 * 4),                # 2 32-row tiles into 32
    (512, 512, 3584, "mmq_kw<q4_K>", 0),                                # K split over waves: no scratch
    (512, 3584, 3584, "mmq<q4_K>", 0),                                  # 448 32-row tiles, none cut
    (100, 306 * 256 - 13, 1024, "mmq_f6<q4_K plane>", 100 * 2 * 128 * 128 * 4),  # 100 tiles into 2
    (40, 256 * 256, 512, "mmq_f6<q4_K plane>", 0),                      # one whole round, nothing cut
]


def run_pair(M, N, K, kernel, cut, seed):
    import torch
    dev = device()
    say(f"gemm_noalloc q4_K M={M} N={N} K={K}")
    raw = weights(mq.Q4_K, N, K, "random", seed)
    W = to_dev(raw.reshape(-1), dev)
    qtype = mq.Q4_K
    if "plane" in kernel:
        W = mq.repack(W, mq.Q4_K, N, K)
        qtype = mq.Q4_K | mq.REPACKED
    X = synth.activations(M, K, config_index=12, tensor_index=seed)
    Xq = mq.quantize_act(to_dev(X, dev))
    need = mq.gemm_scratch_bytes(qtype, M, N, K)
    assert need >= cut and need - cut < 4096
    Y_ref = mq.gemm(W, qtype, Xq, M, N, K)
    assert mq.last_kernel() == kernel, mq.last_kernel()
    Y = torch.full((M, N), float("nan"), dtype=torch.float32, device=dev)
    mq.gemm_noalloc(W, qtype, Xq, M, N, K, Y)
    assert mq.last_kernel() == kernel, mq.last_kernel()
    torch.cuda.synchronize()
    a, b = Y.cpu().numpy(), Y_ref.cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), \
        f"M={M} N={N} K={K}: {np.count_nonzero(a.view(np.uint32) != b.view(np.uint32))} elements differ"


def test_noalloc_matches_gemm_over_calls_in_a_row():
    mq.init(0)
    for i, case in enumerate(CASES):
        run_pair(*case, seed=200 + i)
    # the first shape again, after the array has held every other call's data
    run_pair(*CASES[0], seed=200)


def test_noalloc_refuses_without_touching_the_device():
    import torch
    dev = device()
    mq.init(0)
    M, N, K = 64, 256, 256
    W = torch.zeros(mq.weight_bytes(mq.Q4_K, N, K), dtype=torch.uint8, device=dev)
    Xq = torch.zeros(mq.act_bytes(M, K), dtype=torch.uint8, device=dev)
    lib = mq.load()
    assert lib.mq_gemm_noalloc(W.data_ptr(), mq.Q4_K, Xq.data_ptr(), None, M, N, K, None) == -1
    assert lib.mq_gemm_noalloc(W.data_ptr(), mq.Q4_K, Xq.data_ptr(), W.data_ptr(), M, N, 100, None) == -2
