// mq_repack: the one-time device-layout transform of a weight matrix ("minfer CUDA
// Backend Design", 2.3 Weight residency and registry: Q6_K is repacked into 16-byte
// aligned 224-byte slots so that its fields can be read with 16-byte loads).
//
// Every in_bytes-byte block of the GGUF payload goes to its own slot_bytes-byte slot at
// byte offset `off`; the other bytes of the slot are zero.  One thread writes one output
// dword (coalesced stores) from the up to four payload bytes it covers (byte loads: the
// GGUF blocks are only 2-byte aligned).
#include "mq_internal.h"

namespace mq {

namespace {

__global__ __launch_bounds__(256) void repack_kernel(const uint8_t* __restrict__ W, uint32_t* __restrict__ Wr,
                                                     int64_t words, int in_bytes, int slot_words, int off) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t o = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; o < words; o += stride) {
        const int64_t slot = o / slot_words;
        const int j0 = 4 * int(o - slot * slot_words) - off;   // block byte of the dword's byte 0
        const uint8_t* blk = W + slot * in_bytes;
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int j = j0 + b;
            if (j >= 0 && j < in_bytes) v |= uint32_t(blk[j]) << (8 * b);
        }
        Wr[o] = v;
    }
}

}  // namespace

hipError_t launch_repack(const uint8_t* W, uint8_t* Wr, int64_t blocks, int in_bytes, int slot_bytes, int off,
                         hipStream_t s) {
    const int slot_words = slot_bytes / 4;
    const int64_t words = blocks * slot_words;
    const int64_t want = (words + 255) / 256;
    const int grid = int(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(repack_kernel, dim3(grid), dim3(256), 0, s, W, reinterpret_cast<uint32_t*>(Wr), words,
                       in_bytes, slot_words, off);
    return hipGetLastError();
}

}  // namespace mq
