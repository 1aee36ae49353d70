// mq_repack: the one-time device-layout transform of a weight matrix ("minfer CUDA
// Backend Design", 2.3 Weight residency and registry: Q6_K is repacked into 16-byte
// aligned 224-byte slots so that its fields can be read with 16-byte loads).
//
// Every in_bytes-byte block of the GGUF payload goes to its own slot_bytes-byte slot at
// byte offset `off`; the other bytes of the slot are zero.  One thread writes one output
// dword (coalesced stores) from the up to four payload bytes it covers (byte loads: the
// GGUF blocks are only 2-byte aligned).
//
// Q4_K goes to the MMQ plane of the fp6 matrix-unit product (layout in mq_internal.h; the
// pre-decoded weight plane of the same page, 2.3): per 64-value step and weight row, each of
// the step's two 32-value sub-blocks as a 24-byte record of its codes c, each the OCP FP6
// E2M3 code of c / 2 (exact), value i at bits 6 i .. 6 i + 5, plus the bf16 hi + lo parts of
// its scale d * sc and of its min -dmin * m laid out as the operands of the kernel's bf16
// scale products.  Rows N..Np-1 are zero.  One thread writes one (step, sub-block, row).
//
// Q4_K's row-tiled layout (for the GEMV of long rows; mq_internal.h) moves whole 144-byte
// blocks: a group of rows stores their super-block 0 blocks one after another, then their
// super-block 1 blocks, and so on.
#include "mmq_common.h"
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

__global__ __launch_bounds__(256) void repack_q4k_plane_kernel(const uint8_t* __restrict__ W,
                                                                uint8_t* __restrict__ Wp, int64_t N, int64_t Np,
                                                                int64_t items, int64_t row_bytes) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t it = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; it < items; it += stride) {
        const int64_t n = it % Np;
        const int64_t su = it / Np;
        const int u = int(su & 1);
        const int64_t step = su >> 1;
        uint32_t rec[6] = {0u, 0u, 0u, 0u, 0u, 0u};
        uint32_t outer0 = 0, outer1 = 0, min0 = 0, min1 = 0;
        if (n < N) {
            const int64_t b = 2 * step + u;   // 32-value sub-block of the row
            const int jb = int(b & 7);
            const uint8_t* blk = W + n * row_bytes + (b >> 3) * 144;
            const uint4 hd = *reinterpret_cast<const uint4*>(blk);
            const uint4* qs = reinterpret_cast<const uint4*>(blk + 16 + 32 * (jb >> 1));
            const uint4 qa = qs[0], qb = qs[1];
            const uint32_t w[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
            const int shift = 4 * (jb & 1);   // even sub-blocks: low nibbles, odd: high
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const uint32_t c6 = e2m3_half_code(int((w[i >> 2] >> (8 * (i & 3) + shift)) & 15u));
                const int bit = 6 * i, wd = bit >> 5, o = bit & 31;
                rec[wd] |= c6 << o;
                if (o > 26) rec[wd + 1] |= c6 >> (32 - o);
            }
            uint32_t sc, mn;
            q4k_scale_min(hd.y, hd.z, hd.w, jb, sc, mn);
            const float d = half_bits_to_float(hd.x & 0xFFFFu), dmin = half_bits_to_float(hd.x >> 16);
            const uint32_t dw = bf16_hilo_bits(d * float(sc));        // exact product
            const uint32_t mw = bf16_hilo_bits(-(dmin * float(mn)));   // exact product
            outer0 = (dw & 0xFFFFu) | (dw << 16);        // dw_hi twice
            outer1 = (dw >> 16) | (dw & 0xFFFF0000u);    // dw_lo twice
            min0 = mw;
            min1 = mw;
        }
        uint8_t* slab = Wp + step * 80 * Np;
        const int64_t r = int64_t(u) * Np + n;
        *reinterpret_cast<uint4*>(slab + r * 16) = make_uint4(rec[0], rec[1], rec[2], rec[3]);
        *reinterpret_cast<uint2*>(slab + 32 * Np + r * 8) = make_uint2(rec[4], rec[5]);
        *reinterpret_cast<uint2*>(slab + 48 * Np + r * 8) = make_uint2(outer0, outer1);
        *reinterpret_cast<uint2*>(slab + 64 * Np + r * 8) = make_uint2(min0, min1);
    }
}

// Q4_K's row-tiled layout: one thread per 16-byte chunk of the output (block chunk c of
// row r of the group, super-block s, group g), copied from the GGUF payload; the filler
// rows of the last group are zero.
__global__ __launch_bounds__(256) void repack_q4k_row_tiled_kernel(const uint4* __restrict__ W, uint4* __restrict__ Wr,
                                                                   int64_t N, int64_t chunks, int SB, int R) {
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t o = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; o < chunks; o += stride) {
        const int64_t blk = o / 9;
        const int c = int(o - blk * 9);
        const int r = int(blk % R);
        const int64_t gs = blk / R;
        const int s = int(gs % SB);
        const int64_t n = (gs / SB) * R + r;
        Wr[o] = n < N ? W[(n * SB + s) * 9 + c] : make_uint4(0u, 0u, 0u, 0u);
    }
}

}  // namespace

hipError_t launch_repack_q4k_row_tiled(const uint8_t* W, uint8_t* Wr, int64_t N, int64_t K, hipStream_t s) {
    const int64_t chunks = int64_t(row_tiled_bytes(N, K) / 16);
    const int64_t want = (chunks + 255) / 256;
    const int grid = int(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(repack_q4k_row_tiled_kernel, dim3(grid), dim3(256), 0, s, reinterpret_cast<const uint4*>(W),
                       reinterpret_cast<uint4*>(Wr), N, chunks, int(K / 256), row_tile_rows(N));
    return hipGetLastError();
}

hipError_t launch_repack_q4k_plane(const uint8_t* W, uint8_t* Wp, int64_t N, int64_t K, hipStream_t s) {
    const int64_t Np = f6_weight_rows(N);
    const int64_t items = act_steps(K) * 2 * Np;
    const int64_t want = (items + 255) / 256;
    const int grid = int(want < 65536 ? want : 65536);
    hipLaunchKernelGGL(repack_q4k_plane_kernel, dim3(grid), dim3(256), 0, s, W, Wp, N, Np, items, (K / 256) * 144);
    return hipGetLastError();
}

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
