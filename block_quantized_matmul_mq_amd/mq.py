"""Thin ctypes binding over libmq.so (C ABI in include/mq.h).

Argument marshalling only: torch tensors in, device pointers and the current
torch stream out; every step of the computation runs in the HIP kernels.
Loading fails loudly when the library has not been built -- there is no host
fallback.  Call ``build()`` (or ``python -m block_quantized_matmul_mq_amd.build``)
first.
"""

import ctypes
import os

Q4_0 = 2
Q4_1 = 3
Q5_0 = 6
Q5_1 = 7
Q8_0 = 8
Q4_K = 12
Q5_K = 13
Q6_K = 14
REPACKED = 0x100   # OR-ed into Q8_0 / Q6_K / Q4_K: weights in the layout mq_repack writes
ROW_TILED = 0x200  # OR-ed into Q4_K: its row-tiled layout (long-row GEMV), from repack(.., Q4_K | ROW_TILED, ..)

MQ_OK = 0
ERRORS = {
    -1: "MQ_ERR_ARG", -2: "MQ_ERR_SHAPE", -3: "MQ_ERR_TYPE", -4: "MQ_ERR_SIZE",
    -5: "MQ_ERR_ALIGN", -6: "MQ_ERR_DEVICE", -7: "MQ_ERR_LAUNCH", -8: "MQ_ERR_NOINIT",
}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmq.so")

# Every symbol include/mq.h declares, with its ctypes signature.
_SIGNATURES = {
    "mq_init": (ctypes.c_int, [ctypes.c_int]),
    "mq_weight_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]),
    "mq_act_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
    "mq_act_scale_offset": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
    "mq_act_sum_offset": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
    "mq_act_f6_offset": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64]),
    "mq_quantize_act": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_void_p]),
    "mq_gemv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "mq_gemm_scratch_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]),
    "mq_gemm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                               ctypes.c_size_t, ctypes.c_void_p]),
    "mq_debug_lds_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int64]),
    "mq_gemm_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "mq_debug_gemm_blockdots": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_void_p]),
    "mq_debug_refuse_launches": (ctypes.c_int, [ctypes.c_int]),
    "mq_repack_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]),
    "mq_repack": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_size_t,
                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mq_device_lds_bytes": (ctypes.c_int, []),
    "mq_last_error": (ctypes.c_char_p, []),
    "mq_last_kernel": (ctypes.c_char_p, []),
    "mq_version": (ctypes.c_char_p, []),
}


class MQError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code


_lib = None


def load():
    """Load libmq.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m block_quantized_matmul_mq_amd.build`")
        # torch first: its bundled HIP runtime then also serves libmq (libmq's dependency
        # on libamdhip64.so.7 resolves to the copy already loaded).  Loaded the other way
        # round, the process would hold two HIP runtimes, and the second one to open the
        # device finds none.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def last_error():
    return load().mq_last_error().decode()


def last_kernel():
    return load().mq_last_kernel().decode()


def _check(code):
    if code != MQ_OK:
        raise MQError(code, last_error())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _nbytes(t):
    return t.numel() * t.element_size()


def _refuse(code, fn, msg):
    raise MQError(code, f"{fn}: {msg}")


def _contiguous(t, fn, name):
    if not t.is_contiguous():
        _refuse(-1, fn, f"{name} must be contiguous")


def _weights(W, qtype, N, K, fn):
    """W must hold exactly the payload of an N x K matrix of qtype (the exact-length gate)."""
    need = weight_bytes(qtype, N, K)
    if need == 0:
        _refuse(-3, fn, f"type {qtype} with N={N} K={K} has no payload size (type or K invalid)")
    _contiguous(W, fn, "W")
    if _nbytes(W) != need:
        _refuse(-4, fn, f"W holds {_nbytes(W)} bytes, an {N} x {K} type-{qtype} payload is exactly {need}")


def _f32(t, numel, fn, name):
    import torch
    if t.dtype != torch.float32:
        _refuse(-1, fn, f"{name} must be float32, not {t.dtype}")
    _contiguous(t, fn, name)
    if t.numel() != numel:
        _refuse(-4, fn, f"{name} has {t.numel()} elements, {numel} expected")


def _buffer(t, min_bytes, fn, name):
    _contiguous(t, fn, name)
    if _nbytes(t) < min_bytes:
        _refuse(-4, fn, f"{name} holds {_nbytes(t)} bytes, {min_bytes} required")


def _same_device(fn, *tensors):
    devs = {(t.device.type, t.device.index) for t in tensors}
    if len(devs) != 1 or next(iter(devs))[0] != "cuda":
        _refuse(-6, fn, f"every tensor must be on one GPU device, got {sorted(map(str, devs))}")


def init(device=0):
    _check(load().mq_init(device))


def weight_bytes(qtype, N, K):
    return load().mq_weight_bytes(qtype, N, K)


def repack_bytes(qtype, N, K):
    return load().mq_repack_bytes(qtype, N, K)


def repack(W, qtype, N, K, Wr=None, stream=None):
    """The repacked layout of a GGUF payload W (uint8 CUDA tensor); use with qtype | REPACKED
    (or, for qtype = Q4_K | ROW_TILED, the row-tiled layout; use with Q4_K | ROW_TILED)."""
    import torch
    _weights(W, qtype & ~ROW_TILED, N, K, "repack")
    need = repack_bytes(qtype, N, K)
    if Wr is None:
        Wr = torch.empty(need, dtype=torch.uint8, device=W.device)
    else:
        _buffer(Wr, need, "repack", "Wr")
    _same_device("repack", W, Wr)
    _check(load().mq_repack(ctypes.c_void_p(W.data_ptr()), qtype, N, K, _nbytes(W),
                            ctypes.c_void_p(Wr.data_ptr()), _nbytes(Wr), _stream(stream)))
    return Wr


def act_bytes(M, K):
    return load().mq_act_bytes(M, K)


def act_layout(M, K):
    """(total bytes, scale offset, sum offset) of the quantized activation plane."""
    lib = load()
    return lib.mq_act_bytes(M, K), lib.mq_act_scale_offset(M, K), lib.mq_act_sum_offset(M, K)


def act_f6(Xq, M, K):
    """View (uint8 [ceil(K/64), 128 * Mp]) of the plane's fp6 section, Mp = M rounded up to 128:
    one slab per 64-value step (layout in include/mq.h)."""
    off = load().mq_act_f6_offset(M, K)
    T = (K + 63) // 64
    Mp = -(-M // 128) * 128
    return Xq[off:off + T * 128 * Mp].view(T, 128 * Mp)


def gemm_scratch_bytes(qtype, M, N, K):
    return load().mq_gemm_scratch_bytes(qtype, M, N, K)


def quantize_act(X, Xq=None, stream=None):
    """X: f32 [M, K] CUDA tensor -> Xq: uint8 plane of act_bytes(M, K) bytes."""
    import torch
    if X.dim() != 2:
        _refuse(-1, "quantize_act", f"X must be 2-D [M, K], not {tuple(X.shape)}")
    M, K = X.shape
    _f32(X, M * K, "quantize_act", "X")
    need = act_bytes(M, K)
    if need == 0:
        _refuse(-2, "quantize_act", f"K={K} is not a positive multiple of 32")
    if Xq is None:
        Xq = torch.empty(need, dtype=torch.uint8, device=X.device)
    else:
        _buffer(Xq, need, "quantize_act", "Xq")
    _same_device("quantize_act", X, Xq)
    _check(load().mq_quantize_act(ctypes.c_void_p(X.data_ptr()), ctypes.c_void_p(Xq.data_ptr()), M, K,
                                  _stream(stream)))
    return Xq


def split_act(Xq, M, K):
    """Views (codes int8 [M, K], scales f32 [M, K/32], sums int32 [M, K/32]) into a plane."""
    import torch
    _, so, uo = act_layout(M, K)
    nb = K // 32
    codes = Xq[:M * K].view(torch.int8).view(M, K)
    scales = Xq[so:so + 4 * M * nb].view(torch.float32).view(M, nb)
    sums = Xq[uo:uo + 4 * M * nb].view(torch.int32).view(M, nb)
    return codes, scales, sums


def gemv(W, qtype, x, N, K, y=None, stream=None):
    """y[N] = deq(W) @ x for a uint8 GGUF payload W and f32 x[K] (CUDA tensors)."""
    import torch
    _weights(W, qtype, N, K, "gemv")
    _f32(x, K, "gemv", "x")
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=x.device)
    else:
        _f32(y, N, "gemv", "y")
    _same_device("gemv", W, x, y)
    _check(load().mq_gemv(ctypes.c_void_p(W.data_ptr()), qtype, ctypes.c_void_p(x.data_ptr()),
                          ctypes.c_void_p(y.data_ptr()), N, K, _stream(stream)))
    return y


def _act_plane(Xq, M, K, fn):
    need = act_bytes(M, K)
    if need == 0:
        _refuse(-2, fn, f"M={M} K={K}: K is not a positive multiple of 32")
    _buffer(Xq, need, fn, "Xq")


def gemm(W, qtype, Xq, M, N, K, Y=None, scratch=None, stream=None):
    """Y[M, N] from a quantized activation plane Xq and weights W (CUDA tensors)."""
    import torch
    _weights(W, qtype, N, K, "gemm")
    _act_plane(Xq, M, K, "gemm")
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=Xq.device)
    else:
        _f32(Y, M * N, "gemm", "Y")
    need = gemm_scratch_bytes(qtype, M, N, K)
    if scratch is None and need:
        scratch = torch.zeros(need, dtype=torch.uint8, device=Xq.device)
    tensors = [W, Xq, Y]
    if scratch is not None:
        _buffer(scratch, need, "gemm", "scratch")
        tensors.append(scratch)
    _same_device("gemm", *tensors)
    sp = ctypes.c_void_p(scratch.data_ptr()) if scratch is not None else ctypes.c_void_p(0)
    sb = _nbytes(scratch) if scratch is not None else 0
    _check(load().mq_gemm(ctypes.c_void_p(W.data_ptr()), qtype, ctypes.c_void_p(Xq.data_ptr()),
                          ctypes.c_void_p(Y.data_ptr()), M, N, K, sp, sb, _stream(stream)))
    return Y


def gemm_noalloc(W, qtype, Xq, M, N, K, Y, stream=None):
    """mq_gemm_noalloc: the product into a caller-provided Y, with the library's own
    per-device scratch (the call allocates nothing; overlapping calls on one device race)."""
    _weights(W, qtype, N, K, "gemm_noalloc")
    _act_plane(Xq, M, K, "gemm_noalloc")
    _f32(Y, M * N, "gemm_noalloc", "Y")
    _same_device("gemm_noalloc", W, Xq, Y)
    _check(load().mq_gemm_noalloc(ctypes.c_void_p(W.data_ptr()), qtype, ctypes.c_void_p(Xq.data_ptr()),
                                  ctypes.c_void_p(Y.data_ptr()), M, N, K, _stream(stream)))
    return Y


def gemm_blockdots(W, qtype, Xq, M, N, K, D=None, stream=None):
    """Exact int32 block dots [M, N, G] of the MMQ kernel (G = K/32, or K/16 for Q6_K)."""
    import torch
    _weights(W, qtype, N, K, "gemm_blockdots")
    _act_plane(Xq, M, K, "gemm_blockdots")
    G = K // 16 if (qtype & ~REPACKED) == Q6_K else K // 32
    if D is None:
        D = torch.empty((M, N, G), dtype=torch.int32, device=Xq.device)
    else:
        if D.dtype != torch.int32:
            _refuse(-1, "gemm_blockdots", f"D must be int32, not {D.dtype}")
        _contiguous(D, "gemm_blockdots", "D")
        if D.numel() != M * N * G:
            _refuse(-4, "gemm_blockdots", f"D has {D.numel()} elements, {M * N * G} expected")
    _same_device("gemm_blockdots", W, Xq, D)
    _check(load().mq_debug_gemm_blockdots(ctypes.c_void_p(W.data_ptr()), qtype, ctypes.c_void_p(Xq.data_ptr()),
                                          ctypes.c_void_p(D.data_ptr()), M, N, K, _stream(stream)))
    return D
