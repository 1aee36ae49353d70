// libmq C ABI: argument validation, device checks and kernel dispatch.
//
// Every entry point validates its arguments before making any HIP call and
// returns a negative MQ_ERR_* code with a message on failure; a refused launch
// is an error, never a fallback to another kernel ("minfer CUDA Backend
// Design", 4.3 Eligibility and 4.9 GPU safety: errors are errors, launch
// returns are read at the call site, device limits are queried at run time).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/mq.h"
#include "mq_internal.h"

namespace mq {

namespace {

thread_local std::string g_error;
thread_local const char* g_last_kernel = "";
thread_local int g_refuse_launches = 0;   // mq_debug_refuse_launches

constexpr int kMaxDevices = 64;
DeviceInfo g_devices[kMaxDevices];

// Scratch of mq_gemm_noalloc: one array per device for the life of the process.  The
// first kNoAllocCounterBytes hold the split-tile counters of both MMQ kernels (at most 256
// cut tiles), which every launch leaves at zero (cleared once, when mq_init first sets up
// the device); the partial tiles follow.  Every valid shape's partials fit: both plans cut
// at most one round of workgroups' worth of tiles (512 partial tiles of 128 x 128
// f32), 32 MiB.
constexpr size_t kNoAllocCounterBytes = 4096;
constexpr size_t kNoAllocPartialBytes = size_t(MQ_NOALLOC_PARTIAL_BYTES);
static __device__ __align__(256) uint8_t noalloc_scratch[kNoAllocCounterBytes + kNoAllocPartialBytes];

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

int block_values(int type) {
    switch (type) {
        case MQ_Q4_0: case MQ_Q4_1: case MQ_Q5_0: case MQ_Q5_1: case MQ_Q8_0: return 32;
        case MQ_Q4_K: case MQ_Q5_K: case MQ_Q6_K: return 256;
        default: return 0;
    }
}

int block_bytes(int type) {
    switch (type) {
        case MQ_Q4_0: return 18;
        case MQ_Q4_1: return 20;
        case MQ_Q5_0: return 22;
        case MQ_Q5_1: return 24;
        case MQ_Q8_0: return 34;
        case MQ_Q4_K: return 144;
        case MQ_Q5_K: return 176;
        case MQ_Q6_K: return 210;
        default: return 0;
    }
}

// The slot a block takes in the layout mq_repack writes, and the block's offset in it:
// Q8_0 36 bytes with the block at 2 (its 32 codes then start 4-byte aligned), Q6_K 224
// bytes with the block at 0 (16-byte aligned slots).  Q4_K's repacked layout is not a slot
// layout but the MMQ plane of the fp6 kernel (kPlane; mq_internal.h).
constexpr int kPlane = -1;
BlockLayout repacked_layout(int base) {
    switch (base) {
        case MQ_Q8_0: return {36, 2};
        case MQ_Q6_K: return {224, 0};
        case MQ_Q4_K: return {kPlane, 0};
        default: return {0, 0};
    }
}
bool is_plane(BlockLayout lay) { return lay.stride == kPlane; }

// A type id is a GGUF type, optionally OR-ed with MQ_REPACKED for the layout mq_repack
// writes, or Q4_K OR-ed with MQ_ROW_TILED for its row-tiled layout.  Returns the GGUF type
// (0 for an unknown id or a type with no such layout) and the layout of its blocks.
int parse_type(int type, BlockLayout& lay) {
    if (type & MQ_ROW_TILED) {
        if (type != (MQ_Q4_K | MQ_ROW_TILED)) return 0;
        lay = BlockLayout{block_bytes(MQ_Q4_K), 0, true};
        return MQ_Q4_K;
    }
    const int base = type & ~MQ_REPACKED;
    if (block_values(base) == 0) return 0;
    if (type & MQ_REPACKED) {
        lay = repacked_layout(base);
        return lay.stride ? base : 0;
    }
    lay = BlockLayout{block_bytes(base), 0};
    return base;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape/type checks shared by the weight-consuming calls (`type` without the repack flag).
int check_weight_shape(const char* fn, int type, int64_t N, int64_t K) {
    if (block_values(type) == 0) return fail(MQ_ERR_TYPE, "%s: unsupported weight type %d", fn, type);
    if (N <= 0 || K <= 0) return fail(MQ_ERR_ARG, "%s: N=%lld K=%lld must be positive", fn, (long long)N, (long long)K);
    if (K % block_values(type) != 0)
        return fail(MQ_ERR_SHAPE, "%s: K=%lld is not a multiple of the %d-value block of type %d", fn,
                    (long long)K, block_values(type), type);
    if (K > MQ_MAX_K || N > MQ_MAX_N)
        return fail(MQ_ERR_SHAPE, "%s: N=%lld K=%lld exceeds the limits N<=%d K<=%d", fn, (long long)N,
                    (long long)K, MQ_MAX_N, MQ_MAX_K);
    return MQ_OK;
}

int check_ready(const char* fn) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(MQ_ERR_DEVICE, "%s: hipGetDevice failed: %s", fn, hipGetErrorName(e));
    if (dev < 0 || dev >= kMaxDevices || !g_devices[dev].ready)
        return fail(MQ_ERR_NOINIT, "%s: mq_init has not succeeded on device %d", fn, dev);
    return MQ_OK;
}

int launch_status(const char* fn, hipError_t e, const char* kernel) {
    g_last_kernel = kernel;
    if (e != hipSuccess)
        return fail(MQ_ERR_LAUNCH, "%s: launch of %s refused: %s", fn, kernel, hipGetErrorName(e));
    return MQ_OK;
}

// mq_debug_refuse_launches: true when this call is to take the refused-launch path (the
// caller then reports hipErrorLaunchFailure without launching)
bool refuse_this_launch() {
    if (g_refuse_launches <= 0) return false;
    --g_refuse_launches;
    return true;
}

}  // namespace

const DeviceInfo* device_info() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    return g_devices[dev].ready ? &g_devices[dev] : nullptr;
}

}  // namespace mq

using namespace mq;

extern "C" {

const char* mq_version(void) { return "libmq 0.1 (gfx950)"; }

const char* mq_last_error(void) { return g_error.c_str(); }

const char* mq_last_kernel(void) { return g_last_kernel; }

int mq_debug_refuse_launches(int count) {
    if (count < 0) return fail(MQ_ERR_ARG, "mq_debug_refuse_launches: count=%d must not be negative", count);
    g_refuse_launches = count;
    return MQ_OK;
}

int mq_device_lds_bytes(void) {
    const DeviceInfo* info = device_info();
    return info ? int(info->lds_per_block) : 0;
}

int mq_init(int device) {
    if (device < 0 || device >= kMaxDevices) return fail(MQ_ERR_ARG, "mq_init: device %d out of range", device);
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count <= 0)
        return fail(MQ_ERR_DEVICE, "mq_init: no HIP device (%s)", hipGetErrorName(e));
    if (device >= count) return fail(MQ_ERR_DEVICE, "mq_init: device %d of %d", device, count);
    e = hipSetDevice(device);
    if (e != hipSuccess) return fail(MQ_ERR_DEVICE, "mq_init: hipSetDevice(%d): %s", device, hipGetErrorName(e));
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, device);
    if (e != hipSuccess)
        return fail(MQ_ERR_DEVICE, "mq_init: hipGetDeviceProperties(%d): %s", device, hipGetErrorName(e));
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
        return fail(MQ_ERR_DEVICE, "mq_init: device %d is %s, this library is built for gfx950 only", device,
                    prop.gcnArchName);
    DeviceInfo& info = g_devices[device];
    info.cu_count = prop.multiProcessorCount;
    // the largest LDS a workgroup may use once its kernel opts in (160 KB on gfx950)
    size_t lds = prop.sharedMemPerBlockOptin;
    if (lds < prop.sharedMemPerBlock) lds = prop.sharedMemPerBlock;
    if (prop.maxSharedMemoryPerMultiProcessor && lds > prop.maxSharedMemoryPerMultiProcessor)
        lds = prop.maxSharedMemoryPerMultiProcessor;
    info.lds_per_block = lds;
    // Kernel attributes are set here, once, so that no call ever sets one inside a stream capture.
    e = gemv_set_attributes(lds);
    if (e == hipSuccess) e = gemv_q8_set_attributes(lds);
    if (e != hipSuccess)
        return fail(MQ_ERR_DEVICE, "mq_init: setting the GEMV LDS limit to %zu bytes failed: %s", lds,
                    hipGetErrorName(e));
    if (!info.noalloc_scratch) {
        // This device's copy of the array: its device address, read with the device current
        // (the array's name in host code is only a handle), and its counters cleared once.
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(noalloc_scratch));
        if (e != hipSuccess || !ptr)
            return fail(MQ_ERR_DEVICE, "mq_init: no device address for the scratch array on device %d: %s", device,
                        hipGetErrorName(e));
        e = hipMemset(ptr, 0, kNoAllocCounterBytes);
        if (e == hipSuccess) e = hipDeviceSynchronize();
        if (e != hipSuccess)
            return fail(MQ_ERR_DEVICE, "mq_init: clearing the scratch counters on device %d failed: %s", device,
                        hipGetErrorName(e));
        info.noalloc_scratch = static_cast<uint8_t*>(ptr);
    }
    info.ready = true;
    return MQ_OK;
}

size_t mq_weight_bytes(int type, int64_t N, int64_t K) {
    BlockLayout lay;
    const int base = parse_type(type, lay);
    if (base == 0) return 0;
    const int bv = block_values(base);
    if (N <= 0 || K <= 0 || K % bv != 0) return 0;
    if (is_plane(lay)) return f6_weight_plane_bytes(N, K);
    if (lay.row_tiled) return row_tiled_k(K) ? row_tiled_bytes(N, K) : 0;
    return size_t(N) * size_t(K / bv) * size_t(lay.stride);
}

size_t mq_repack_bytes(int type, int64_t N, int64_t K) {
    if (type & MQ_REPACKED) return 0;
    if (type & MQ_ROW_TILED) return mq_weight_bytes(type, N, K);
    return mq_weight_bytes(type | MQ_REPACKED, N, K);
}

size_t mq_act_bytes(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0 || K % 32 != 0) return 0;
    return act_bytes(M, K);
}

size_t mq_act_scale_offset(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0 || K % 32 != 0) return 0;
    return act_scale_offset(M, K);
}

size_t mq_act_sum_offset(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0 || K % 32 != 0) return 0;
    return act_sum_offset(M, K);
}

size_t mq_act_f6_offset(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0 || K % 32 != 0) return 0;
    return act_f6_offset(M, K);
}

size_t mq_gemm_scratch_bytes(int type, int64_t M, int64_t N, int64_t K) {
    BlockLayout lay;
    type = parse_type(type, lay);
    if (type == 0) return 0;
    if (M <= 0 || N <= 0 || K <= 0 || M > MQ_MAX_M || N > MQ_MAX_N || K > MQ_MAX_K) return 0;
    if (K % block_values(type) != 0) return 0;
    if (lay.row_tiled) return 0;   // mq_gemm refuses the row-tiled layout
    if (is_plane(lay)) return mmq_f6_scratch_bytes(M, N, K);
    return mmq_scratch_bytes(type, M, N, K);
}

int mq_quantize_act(const float* X, void* Xq, int64_t M, int64_t K, void* stream) {
    const char* fn = "mq_quantize_act";
    if (!X || !Xq) return fail(MQ_ERR_ARG, "%s: null pointer (X=%p Xq=%p)", fn, (const void*)X, Xq);
    if (M <= 0 || K <= 0) return fail(MQ_ERR_ARG, "%s: M=%lld K=%lld must be positive", fn, (long long)M, (long long)K);
    if (K % 32 != 0) return fail(MQ_ERR_SHAPE, "%s: K=%lld is not a multiple of 32", fn, (long long)K);
    if (K > MQ_MAX_K || M > MQ_MAX_M)
        return fail(MQ_ERR_SHAPE, "%s: M=%lld K=%lld exceeds M<=%d K<=%d", fn, (long long)M, (long long)K, MQ_MAX_M, MQ_MAX_K);
    if (!aligned(X, 16) || !aligned(Xq, 256))
        return fail(MQ_ERR_ALIGN, "%s: X must be 16-byte and Xq 256-byte aligned (X=%p Xq=%p)", fn, (const void*)X, Xq);
    int rc = check_ready(fn);
    if (rc) return rc;
    uint8_t* base = static_cast<uint8_t*>(Xq);
    if (refuse_this_launch()) return launch_status(fn, hipErrorLaunchFailure, "quantize_act");
    hipError_t e = launch_quantize_act(X, reinterpret_cast<int8_t*>(base),
                                       reinterpret_cast<float*>(base + act_scale_offset(M, K)),
                                       reinterpret_cast<int32_t*>(base + act_sum_offset(M, K)),
                                       base + act_f6_offset(M, K), M, K, static_cast<hipStream_t>(stream));
    return launch_status(fn, e, "quantize_act");
}

int mq_gemv(const void* W, int type, const float* x, float* y, int64_t N, int64_t K, void* stream) {
    const char* fn = "mq_gemv";
    if (!W || !x || !y) return fail(MQ_ERR_ARG, "%s: null pointer (W=%p x=%p y=%p)", fn, W, (const void*)x, (void*)y);
    BlockLayout lay;
    const int base = parse_type(type, lay);
    if (base == 0) return fail(MQ_ERR_TYPE, "%s: unsupported weight type %d", fn, type);
    if (is_plane(lay))
        return fail(MQ_ERR_TYPE, "%s: type %d is the Q4_K MMQ plane, which only mq_gemm reads (decode the GGUF "
                    "payload itself)", fn, type);
    type = base;
    int rc = check_weight_shape(fn, type, N, K);
    if (rc) return rc;
    if (!aligned(W, 16) || !aligned(x, 16) || !aligned(y, 4))
        return fail(MQ_ERR_ALIGN, "%s: W and x must be 16-byte, y 4-byte aligned (W=%p x=%p y=%p)", fn, W,
                    (const void*)x, (void*)y);
    if (lay.row_tiled && !row_tiled_k(K))
        return fail(MQ_ERR_SHAPE, "%s: the row-tiled Q4_K layout holds rows of more than 16 super-blocks (K > "
                    "4096), not K=%lld", fn, (long long)K);
    rc = check_ready(fn);
    if (rc) return rc;
    if (lay.row_tiled) {
        const char* kernel = "gemv_mfma_long<q4_K row-tiled>";
        if (refuse_this_launch()) return launch_status(fn, hipErrorLaunchFailure, kernel);
        hipError_t e = launch_gemv_row_tiled(static_cast<const uint8_t*>(W), x, y, N, K,
                                             static_cast<hipStream_t>(stream), &kernel);
        return launch_status(fn, e, kernel);
    }
    if (gemv_tile_units(type, K, device_info()->lds_per_block) <= 0)
        return fail(MQ_ERR_SHAPE, "%s: K=%lld does not fit the %zu-byte LDS of this device", fn, (long long)K,
                    device_info()->lds_per_block);
    const char* kernel = "gemv";
    if (refuse_this_launch()) return launch_status(fn, hipErrorLaunchFailure, "gemv");
    hipError_t e = launch_gemv(type, lay, static_cast<const uint8_t*>(W), x, y, N, K,
                               static_cast<hipStream_t>(stream), &kernel);
    return launch_status(fn, e, kernel);
}

static int gemm_common(const char* fn, const void* W, int type, const void* Xq, float* Y, int32_t* D,
                       void* scratch, unsigned* counters, int64_t M, int64_t N, int64_t K, void* stream) {
    if (!W || !Xq || (!Y && !D))
        return fail(MQ_ERR_ARG, "%s: null pointer (W=%p Xq=%p out=%p)", fn, W, Xq, Y ? (void*)Y : (void*)D);
    BlockLayout lay;
    const int base = parse_type(type, lay);
    if (base == 0) return fail(MQ_ERR_TYPE, "%s: unsupported weight type %d", fn, type);
    if (lay.row_tiled)
        return fail(MQ_ERR_TYPE, "%s: type %d is Q4_K's row-tiled layout, which only mq_gemv reads (the prefill "
                    "product reads the GGUF payload or the MMQ plane)", fn, type);
    type = base;
    int rc = check_weight_shape(fn, type, N, K);
    if (rc) return rc;
    if (M <= 0) return fail(MQ_ERR_ARG, "%s: M=%lld must be positive", fn, (long long)M);
    if (M > MQ_MAX_M) return fail(MQ_ERR_SHAPE, "%s: M=%lld exceeds %d", fn, (long long)M, MQ_MAX_M);
    const int64_t groups = type == MQ_Q6_K ? K / 16 : K / 32;
    if (D && int64_t(M) * N * groups > (int64_t(1) << 32))
        return fail(MQ_ERR_SHAPE, "%s: block-dot export of M=%lld N=%lld K=%lld is too large", fn, (long long)M,
                    (long long)N, (long long)K);
    if (!aligned(W, 16) || !aligned(Xq, 256) || (Y && !aligned(Y, 4)) || (D && !aligned(D, 4)))
        return fail(MQ_ERR_ALIGN, "%s: W 16-byte, Xq 256-byte, outputs 4-byte alignment required", fn);
    rc = check_ready(fn);
    if (rc) return rc;
    const uint8_t* xq = static_cast<const uint8_t*>(Xq);
    const char* kernel = "mmq";
    float* Yout = Y;
    if (is_plane(lay)) {
        if (refuse_this_launch()) return launch_status(fn, hipErrorLaunchFailure, "mmq_f6<q4_K plane>");
        hipError_t e = launch_mmq_f6(static_cast<const uint8_t*>(W), xq + act_f6_offset(M, K), Y, D, scratch, counters,
                                     M, N, K, static_cast<hipStream_t>(stream), &kernel);
        return launch_status(fn, e, kernel);
    }
    if (refuse_this_launch()) return launch_status(fn, hipErrorLaunchFailure, "mmq");
    hipError_t e = launch_mmq(type, lay, static_cast<const uint8_t*>(W), reinterpret_cast<const int8_t*>(xq),
                              reinterpret_cast<const float*>(xq + act_scale_offset(M, K)),
                              reinterpret_cast<const int32_t*>(xq + act_sum_offset(M, K)), Yout, D, scratch,
                              counters, M, N, K, static_cast<hipStream_t>(stream), &kernel);
    return launch_status(fn, e, kernel);
}

int mq_gemm(const void* W, int type, const void* Xq, float* Y, int64_t M, int64_t N, int64_t K, void* scratch,
            size_t scratch_bytes, void* stream) {
    const char* fn = "mq_gemm";
    if (!Y) return fail(MQ_ERR_ARG, "%s: null Y", fn);
    const size_t need = mq_gemm_scratch_bytes(type, M, N, K);
    if (scratch_bytes < need || (need && !scratch))
        return fail(MQ_ERR_SIZE, "%s: scratch of %zu bytes at %p, %zu required", fn, scratch_bytes, scratch, need);
    if (need && !aligned(scratch, 16))
        return fail(MQ_ERR_ALIGN, "%s: scratch must be 16-byte aligned (%p)", fn, scratch);
    return gemm_common(fn, W, type, Xq, Y, nullptr, need ? scratch : nullptr, nullptr, M, N, K, stream);
}

int mq_gemm_noalloc(const void* W, int type, const void* Xq, float* Y, int64_t M, int64_t N, int64_t K,
                    void* stream) {
    const char* fn = "mq_gemm_noalloc";
    if (!Y) return fail(MQ_ERR_ARG, "%s: null Y", fn);
    if (mq_gemm_scratch_bytes(type, M, N, K) != 0) {   // a valid shape whose plan cuts tiles
        BlockLayout lay;
        const int base = parse_type(type, lay);
        const size_t need = is_plane(lay) ? mmq_f6_partial_bytes(M, N, K) : mmq_partial_bytes(base, M, N, K);
        if (need > kNoAllocPartialBytes)
            return fail(MQ_ERR_SIZE, "%s: M=%lld N=%lld K=%lld needs %zu bytes of partial tiles, the limit is %zu", fn,
                        (long long)M, (long long)N, (long long)K, need, kNoAllocPartialBytes);
    }
    int rc = check_ready(fn);
    if (rc) return rc;
    uint8_t* base = device_info()->noalloc_scratch;
    return gemm_common(fn, W, type, Xq, Y, nullptr, base + kNoAllocCounterBytes, reinterpret_cast<unsigned*>(base),
                       M, N, K, stream);
}

size_t mq_debug_lds_bytes(int what, int type, int64_t K) {
    BlockLayout lay;
    type = parse_type(type, lay);
    if (type == 0) return 0;
    switch (what) {
        case MQ_LDS_GEMV_FIXED:
            if (K <= 0 || K > MQ_MAX_K || K % block_values(type) != 0) return 0;
            return fixed_lds_bytes(type, K);
        case MQ_LDS_GEMV_TILE_UNITS:
            if (K <= 0 || K > MQ_MAX_K || K % block_values(type) != 0) return 0;
            return size_t(gemv_tile_units(type, K, MQ_GFX950_LDS_BYTES));
        case MQ_LDS_MMQ_I8_BM128: return mmq_smem_bytes(type, 128);
        case MQ_LDS_MMQ_I8_BM32: return mmq_smem_bytes(type, 32);
        case MQ_LDS_MMQ_F6: return type == MQ_Q4_K ? mmq_f6_lds_bytes() : 0;
        case MQ_LDS_MMQ_KW: return type == MQ_Q4_K ? mmq_kw_lds_bytes() : 0;
        default: return 0;
    }
}

int mq_debug_gemm_blockdots(const void* W, int type, const void* Xq, int32_t* D, int64_t M, int64_t N, int64_t K,
                            void* stream) {
    const char* fn = "mq_debug_gemm_blockdots";
    if (!D) return fail(MQ_ERR_ARG, "%s: null D", fn);
    return gemm_common(fn, W, type, Xq, nullptr, D, nullptr, nullptr, M, N, K, stream);
}

int mq_repack(const void* W, int type, int64_t N, int64_t K, size_t nbytes, void* Wr, size_t wr_bytes,
              void* stream) {
    const char* fn = "mq_repack";
    if (!W || !Wr) return fail(MQ_ERR_ARG, "%s: null pointer (W=%p Wr=%p)", fn, W, Wr);
    if (type & MQ_REPACKED) return fail(MQ_ERR_TYPE, "%s: type %d is already the repacked layout", fn, type);
    const bool row_tiled = (type & MQ_ROW_TILED) != 0;
    if (row_tiled) {
        if (type != (MQ_Q4_K | MQ_ROW_TILED)) return fail(MQ_ERR_TYPE, "%s: only Q4_K has a row-tiled layout", fn);
        type = MQ_Q4_K;
        const int rc = check_weight_shape(fn, type, N, K);
        if (rc) return rc;
        if (!row_tiled_k(K))
            return fail(MQ_ERR_SHAPE, "%s: the row-tiled Q4_K layout holds rows of more than 16 super-blocks (K > "
                        "4096), not K=%lld", fn, (long long)K);
    }
    if (block_values(type) != 0 && repacked_layout(type).stride == 0)
        return fail(MQ_ERR_TYPE, "%s: type %d has no repacked layout", fn, type);
    int rc = check_weight_shape(fn, type, N, K);
    if (rc) return rc;
    const size_t in_bytes = mq_weight_bytes(type, N, K);
    const size_t out_bytes = row_tiled ? row_tiled_bytes(N, K) : mq_repack_bytes(type, N, K);
    if (nbytes != in_bytes)
        return fail(MQ_ERR_SIZE, "%s: payload of %zu bytes, a %lld x %lld type-%d matrix is exactly %zu", fn, nbytes,
                    (long long)N, (long long)K, type, in_bytes);
    if (wr_bytes < out_bytes)
        return fail(MQ_ERR_SIZE, "%s: output of %zu bytes, %zu required", fn, wr_bytes, out_bytes);
    if (!aligned(W, 16) || !aligned(Wr, 16))
        return fail(MQ_ERR_ALIGN, "%s: W and Wr must be 16-byte aligned (W=%p Wr=%p)", fn, W, Wr);
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(W), a1 = a0 + in_bytes;
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(Wr), b1 = b0 + out_bytes;
    if (a0 < b1 && b0 < a1) return fail(MQ_ERR_ARG, "%s: W and Wr overlap", fn);
    rc = check_ready(fn);
    if (rc) return rc;
    if (row_tiled) {
        if (refuse_this_launch()) return launch_status(fn, hipErrorLaunchFailure, "repack");
        hipError_t e = launch_repack_q4k_row_tiled(static_cast<const uint8_t*>(W), static_cast<uint8_t*>(Wr), N, K,
                                                   static_cast<hipStream_t>(stream));
        return launch_status(fn, e, "repack");
    }
    const BlockLayout lay = repacked_layout(type);
    if (is_plane(lay)) {
        if (refuse_this_launch()) return launch_status(fn, hipErrorLaunchFailure, "repack");
        hipError_t e = launch_repack_q4k_plane(static_cast<const uint8_t*>(W), static_cast<uint8_t*>(Wr), N, K,
                                               static_cast<hipStream_t>(stream));
        return launch_status(fn, e, "repack");
    }
    const int64_t blocks = N * (K / block_values(type));
    if (refuse_this_launch()) return launch_status(fn, hipErrorLaunchFailure, "repack");
    hipError_t e = launch_repack(static_cast<const uint8_t*>(W), static_cast<uint8_t*>(Wr), blocks, block_bytes(type),
                                 lay.stride, lay.off, static_cast<hipStream_t>(stream));
    return launch_status(fn, e, "repack");
}

}  // extern "C"
