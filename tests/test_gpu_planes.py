"""GPU parity of the Q4_K MMQ plane (mq_repack of Q4_K) and of the fp6 section of the
quantized activation plane, and of mq_gemm on the plane (the fp6 matrix-unit kernel):

* the plane bytes mq_repack writes equal the oracle's ``q4_k_plane`` bit for bit, and
  the fp6 section mq_quantize_act writes equals ``act_f6_section`` bit for bit;
* the block dots the kernel forms (exported by the same kernel template) equal the
  oracle's int block dots bit for bit;
* Y is within 2e-4 of the oracle's f64 product (normalized per element), on ragged
  shapes, K-split shapes and the full 7B ffn_up product (sampled columns).
"""

import numpy as np
import pytest

import oracle
from block_quantized_matmul_mq_amd import mq, synth

from gpu_cases import check_normalized, device, row_norms, say, to_dev, weights

pytestmark = pytest.mark.gpu

Q4K = mq.Q4_K
PLANE = mq.Q4_K | mq.REPACKED
KERNEL = "mmq_f6<q4_K plane>"


def plane(raw, N, K, dev):
    import torch
    Wp = mq.repack(to_dev(raw.reshape(-1), dev), Q4K, N, K)
    torch.cuda.synchronize()
    assert mq.last_kernel() == "repack"
    return Wp


def act_plane(X, dev):
    import torch
    Xq = mq.quantize_act(to_dev(X, dev))
    torch.cuda.synchronize()
    return Xq


@pytest.mark.parametrize("N,K,kind", [(1, 256, "random"), (37, 512, "random"), (300, 2304, "quantized"),
                                      (1029, 3584, "random")])
def test_plane_bytes_equal_the_oracle(N, K, kind):
    dev = device()
    say(f"plane N={N} K={K} {kind}")
    raw = weights(Q4K, N, K, kind, N)
    got = plane(raw, N, K, dev).cpu().numpy()
    ref = oracle.q4_k_plane(raw, N, K)
    assert got.size == ref.size == mq.repack_bytes(Q4K, N, K)
    assert np.array_equal(got, ref), f"first difference at byte {int(np.argmax(got != ref))}"


def _extreme(M, K, seed):
    X = synth.activations(M, K, config_index=14, tensor_index=seed)
    X[0, :64] = 0.0                                   # zero blocks: scale 0, codes 0
    X[-1, 3::97] = 50.0                               # outliers: codes of +-127
    X[M // 2, 32:64] = np.float32(1e-30)              # a tiny block
    X[M // 2, 96:128] = -2.5                          # a constant block: every code -127
    return X


@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (40, 1024), (130, 3584), (257, 416)])
def test_activation_fp6_section_equals_the_oracle(M, K):
    dev = device()
    say(f"fp6 section M={M} K={K}")
    X = _extreme(M, K, M) if M > 2 else synth.activations(M, K, config_index=14, tensor_index=M)
    Xq = act_plane(X, dev)
    got = mq.act_f6(Xq, M, K).cpu().numpy().reshape(-1)
    q, d, S = oracle.quantize_act(X)
    ref = oracle.act_f6_section(q, d, S)
    assert np.array_equal(got, ref), f"first difference at byte {int(np.argmax(got != ref))}"


def check_plane_product(raw, X, N, K, cols=None, what="", dots=False):
    import torch
    dev = device()
    M = X.shape[0]
    say(f"plane gemm M={M} N={N} K={K} {what}")
    Wp = plane(raw, N, K, dev)
    Xq = act_plane(X, dev)
    q, d, _ = oracle.quantize_act(X)
    if dots:
        D = mq.gemm_blockdots(Wp, PLANE, Xq, M, N, K)
        torch.cuda.synchronize()
        assert mq.last_kernel() == KERNEL
        ref = oracle.block_dots(raw, Q4K, q, N, K)
        got = D.cpu().numpy()
        assert np.array_equal(got, ref), f"{what}: block dots differ at {np.argwhere(got != ref)[:5]}"
    Y = mq.gemm(Wp, PLANE, Xq, M, N, K)
    torch.cuda.synchronize()
    assert mq.last_kernel() == KERNEL
    cols = np.arange(N) if cols is None else cols
    xh = (q.reshape(M, -1, 32).astype(np.float64) * d[..., None].astype(np.float64)).reshape(M, K)
    Y_ref = oracle.mmq(raw.reshape(N, -1)[cols], Q4K, q, d, len(cols), K)
    return check_normalized(Y.cpu().numpy()[:, cols], Y_ref, row_norms(raw, Q4K, N, K, cols),
                            np.linalg.norm(xh, axis=1), f"plane M={M} {N}x{K} {what}")


@pytest.mark.parametrize("kind", ["quantized", "random"])
def test_plane_product_small_ragged(kind):
    # tiles of 128 x 128: ragged M and N everywhere, one tile and several, and K-split plans
    for i, (M, N, K) in enumerate([(1, 1, 256), (3, 33, 512), (37, 130, 1024), (130, 300, 2560),
                                   (129, 257, 1024), (200, 1000, 3584)]):
        raw = weights(Q4K, N, K, kind, 140 + i)
        X = synth.activations(M, K, config_index=14, tensor_index=20 + i)
        check_plane_product(raw, X, N, K, what=kind, dots=True)


def test_plane_product_extreme_activations():
    M, N, K = 130, 300, 1024
    raw = weights(Q4K, N, K, "random", 150)
    check_plane_product(raw, _extreme(M, K, 7), N, K, what="extreme activations", dots=True)


def test_plane_split_k_uneven_ranges():
    # one output tile and a long K: cut into many uneven ranges, summed in range order by the
    # range that finishes last
    M, N, K = 40, 100, 8192
    assert mq.gemm_scratch_bytes(PLANE, M, N, K) > 0
    raw = weights(Q4K, N, K, "random", 151)
    X = synth.activations(M, K, config_index=14, tensor_index=40)
    check_plane_product(raw, X, N, K, what="split-K", dots=True)


def test_plane_whole_tiles_plus_split_tail():
    # 520 tiles of 128 x 128: 512 whole, the last 8 cut into K ranges; sampled columns of both
    M, N, K = 100, 128 * 520, 512
    assert mq.gemm_scratch_bytes(PLANE, M, N, K) > 0
    raw = weights(Q4K, N, K, "quantized", 152)
    X = synth.activations(M, K, config_index=14, tensor_index=41)
    rng = np.random.default_rng(6)
    cols = np.sort(np.concatenate([rng.choice(N - 1024, 200, replace=False), np.arange(N - 1024, N)]))
    check_plane_product(raw, X, N, K, cols=cols, what="whole + split tiles")


def test_plane_full_7b_ffn_up_sampled():
    # the 7B prefill ffn_up product (M = 512, 18944 x 3584, 592 tiles: 80 of them K-split),
    # in the launch configuration the benchmark times; columns sampled from every tile
    M, N, K = 512, 18944, 3584
    raw = synth.quantized_weight(Q4K, N, K, 3, 0)
    X = synth.activations(M, K, 3)
    rng = np.random.default_rng(8)
    cols = np.sort(np.concatenate([np.arange(n0, N, 256) for n0 in (0, 255)] + [rng.choice(N, 200, replace=False)]))
    cols = np.unique(cols)
    check_plane_product(raw, X, N, K, cols=cols, what="7B ffn_up")


def test_plane_matches_the_gguf_path():
    # the same product on the GGUF payload (int8 kernel) agrees within the tolerance
    import torch
    dev = device()
    M, N, K = 300, 4096, 2048
    raw = weights(Q4K, N, K, "quantized", 153)
    X = synth.activations(M, K, config_index=14, tensor_index=42)
    Xq = act_plane(X, dev)
    Y_gguf = mq.gemm(to_dev(raw.reshape(-1), dev), Q4K, Xq, M, N, K)
    Y_plane = mq.gemm(plane(raw, N, K, dev), PLANE, Xq, M, N, K)
    torch.cuda.synchronize()
    q, d, _ = oracle.quantize_act(X)
    xh = (q.reshape(M, -1, 32).astype(np.float64) * d[..., None].astype(np.float64)).reshape(M, K)
    check_normalized(Y_plane.cpu().numpy(), Y_gguf.cpu().numpy().astype(np.float64), row_norms(raw, Q4K, N, K),
                     np.linalg.norm(xh, axis=1), "plane vs GGUF path")
