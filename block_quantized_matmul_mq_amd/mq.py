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
REPACKED = 0x100   # OR-ed into Q8_0 / Q6_K: weights in the layout mq_repack writes

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
    "mq_quantize_act": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_void_p]),
    "mq_gemv": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p]),
    "mq_gemm_scratch_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]),
    "mq_gemm": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                               ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                               ctypes.c_size_t, ctypes.c_void_p]),
    "mq_debug_gemm_blockdots": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_void_p]),
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


def init(device=0):
    _check(load().mq_init(device))


def weight_bytes(qtype, N, K):
    return load().mq_weight_bytes(qtype, N, K)


def repack_bytes(qtype, N, K):
    return load().mq_repack_bytes(qtype, N, K)


def repack(W, qtype, N, K, Wr=None, stream=None):
    """The repacked layout of a GGUF payload W (uint8 CUDA tensor); use with qtype | REPACKED."""
    import torch
    if Wr is None:
        Wr = torch.empty(repack_bytes(qtype, N, K), dtype=torch.uint8, device=W.device)
    _check(load().mq_repack(ctypes.c_void_p(W.data_ptr()), qtype, N, K, W.numel() * W.element_size(),
                            ctypes.c_void_p(Wr.data_ptr()), Wr.numel() * Wr.element_size(), _stream(stream)))
    return Wr


def act_bytes(M, K):
    return load().mq_act_bytes(M, K)


def act_layout(M, K):
    """(total bytes, scale offset, sum offset) of the quantized activation plane."""
    lib = load()
    return lib.mq_act_bytes(M, K), lib.mq_act_scale_offset(M, K), lib.mq_act_sum_offset(M, K)


def gemm_scratch_bytes(qtype, M, N, K):
    return load().mq_gemm_scratch_bytes(qtype, M, N, K)


def quantize_act(X, Xq=None, stream=None):
    """X: f32 [M, K] CUDA tensor -> Xq: uint8 plane of act_bytes(M, K) bytes."""
    import torch
    M, K = X.shape
    if Xq is None:
        Xq = torch.empty(act_bytes(M, K), dtype=torch.uint8, device=X.device)
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
    if y is None:
        y = torch.empty(N, dtype=torch.float32, device=x.device)
    _check(load().mq_gemv(ctypes.c_void_p(W.data_ptr()), qtype, ctypes.c_void_p(x.data_ptr()),
                          ctypes.c_void_p(y.data_ptr()), N, K, _stream(stream)))
    return y


def gemm(W, qtype, Xq, M, N, K, Y=None, scratch=None, stream=None):
    """Y[M, N] from a quantized activation plane Xq and weights W (CUDA tensors)."""
    import torch
    if Y is None:
        Y = torch.empty((M, N), dtype=torch.float32, device=Xq.device)
    need = gemm_scratch_bytes(qtype, M, N, K)
    if scratch is None and need:
        scratch = torch.empty(need, dtype=torch.uint8, device=Xq.device)
    sp = ctypes.c_void_p(scratch.data_ptr()) if scratch is not None else ctypes.c_void_p(0)
    sb = scratch.numel() * scratch.element_size() if scratch is not None else 0
    _check(load().mq_gemm(ctypes.c_void_p(W.data_ptr()), qtype, ctypes.c_void_p(Xq.data_ptr()),
                          ctypes.c_void_p(Y.data_ptr()), M, N, K, sp, sb, _stream(stream)))
    return Y


def gemm_blockdots(W, qtype, Xq, M, N, K, D=None, stream=None):
    """Exact int32 block dots [M, N, G] of the MMQ kernel (G = K/32, or K/16 for Q6_K)."""
    import torch
    G = K // 16 if (qtype & ~REPACKED) == Q6_K else K // 32
    if D is None:
        D = torch.empty((M, N, G), dtype=torch.int32, device=Xq.device)
    _check(load().mq_debug_gemm_blockdots(ctypes.c_void_p(W.data_ptr()), qtype, ctypes.c_void_p(Xq.data_ptr()),
                                          ctypes.c_void_p(D.data_ptr()), M, N, K, _stream(stream)))
    return D
