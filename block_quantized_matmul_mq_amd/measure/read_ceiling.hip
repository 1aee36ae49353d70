// Measurement helper, not part of libmq: a plain streaming read of a device buffer.
//
// It gives the HBM read rate that a kernel of a given launch geometry reaches when all
// it does is read: each lane loads 16-byte chunks, four in flight, in a grid-stride loop
// and folds them into one word, and each wave stores its word (so the loads are live).
// A weight-streaming GEMV moving the same bytes with the same number of workgroups can at
// best match it; the difference to the 8 TB/s of the HBM is launch ramp, tail and the
// memory system, not the GEMV.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__global__ __launch_bounds__(1024) void read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                    uint32_t* __restrict__ sink) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= (a.x ^ a.y ^ a.z ^ a.w) ^ (b.x ^ b.y ^ b.z ^ b.w) ^ (c.x ^ c.y ^ c.z ^ c.w) ^
               (d.x ^ d.y ^ d.z ^ d.w);
    }
    for (; i < n16; i += stride) {
        const uint4 a = p[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if ((threadIdx.x & 63) == 0) sink[int64_t(blockIdx.x) * (blockDim.x / 64) + threadIdx.x / 64] = acc;
}

}  // namespace

extern "C" {

// Words `sink` must hold for a launch of `grid` workgroups of `threads` threads.
size_t mq_measure_sink_words(int grid, int threads) { return size_t(grid) * size_t(threads / 64); }

// Read `bytes` (a multiple of 16) of device memory at `buf` (16-byte aligned) with `grid`
// workgroups of `threads` (64..1024, a multiple of 64) on `stream`.  0 on success, -1 for
// bad arguments, -7 when the launch is refused.
int mq_measure_read(const void* buf, size_t bytes, void* sink, int grid, int threads, void* stream) {
    if (!buf || !sink || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15) || grid <= 0 || threads < 64 ||
        threads > 1024 || threads % 64)
        return -1;
    hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(threads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4*>(buf), int64_t(bytes / 16), static_cast<uint32_t*>(sink));
    return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
