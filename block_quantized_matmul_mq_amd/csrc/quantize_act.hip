// mq_quantize_act kernel: f32 rows -> q8 blocks of 32 with an f32 scale.
//
// Per 32-value block ("minfer Architecture Execution Plan", C4 S2b design
// decision 4: amax, scale amax / 127, round half to even; the scale is kept in
// f32 here):  amax = max |x|;  d = amax / 127 (IEEE f32 division);
// q = clamp(rint(x / d), -127, 127) with a true division, q = 0 when d == 0;
// sum = sum of the 32 codes.
//
// Eight lanes own one block, four values each (one 16-byte load per lane), so
// a wave quantizes eight blocks and the block reductions are three xor
// shuffles.  A wave takes the same block of eight consecutive rows, and a
// workgroup four consecutive blocks of those rows: each wave's stores of the
// row-major arrays below then fill whole 64- or 128-byte segments.  The kernel
// streams X once: it is HBM-bound.
//
// It also writes the fp6 section of the plane (the operands of the fp6 matrix-unit
// product; layout in mq_internal.h): each code as q = 16 h + l with h = q >> 4 in [-8, 7]
// and l = q & 15, as
// the OCP FP6 E2M3 codes of h / 2 and of l / 2 (exact: every multiple of 1/2 up to 7.5 is
// an E2M3 value).  The block's 32 codes of each digit form a 24-byte record, value i in bits
// 6 i .. 6 i + 5 (little endian): lane j of the block packs its four values into bits
// 24 j .. 24 j + 23 and lanes 0..5 assemble one dword each from their neighbours' bits.
// With them go the bf16 operands of the scale products: dx as hi + lo, and tx = dx * S
// (f32 product) as hi + lo.  Rows M..Mp-1 of the section are written as zeros.
#include "mmq_common.h"
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

// a * b rounded to f32: never contracted with the subtraction of the hi/lo split that
// consumes it (tx is defined as the rounded product)
__device__ __forceinline__ float product_f32(float a, float b) {
#pragma clang fp contract(off)
    return a * b;
}

__global__ __launch_bounds__(256) void quantize_act_kernel(const float4* __restrict__ X,
                                                           uint32_t* __restrict__ codes,
                                                           float* __restrict__ scales,
                                                           int32_t* __restrict__ sums,
                                                           uint32_t* __restrict__ f6, int64_t M, int64_t Mp,
                                                           int KB, int block_groups) {
    // workgroup: rows 8 rg .. 8 rg + 7 (of Mp) x blocks 4 bg .. 4 bg + 3; wave w: block 4 bg + w
    const int64_t rg = blockIdx.x / block_groups;
    const int bg = int(blockIdx.x % block_groups);
    const int j = int(threadIdx.x & 7);
    const int64_t m = 8 * rg + ((threadIdx.x >> 3) & 7);
    const int kb = 4 * bg + int(threadIdx.x >> 6);
    const bool in_k = kb < KB;
    const bool live = in_k && m < M;   // rows M..Mp-1 only get the fp6 section's zeros
    const int64_t blk = m * KB + kb;
    const int64_t t = blk * 8 + j;     // this lane's quad of X and of the codes
    const float4 v = live ? X[t] : make_float4(0.f, 0.f, 0.f, 0.f);

    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = fmaxf(a, __shfl_xor(a, 1, 64));
    a = fmaxf(a, __shfl_xor(a, 2, 64));
    a = fmaxf(a, __shfl_xor(a, 4, 64));
    const float d = a / 127.0f;

    int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    if (d > 0.0f) {
        q0 = static_cast<int>(fminf(fmaxf(rintf(v.x / d), -127.0f), 127.0f));
        q1 = static_cast<int>(fminf(fmaxf(rintf(v.y / d), -127.0f), 127.0f));
        q2 = static_cast<int>(fminf(fmaxf(rintf(v.z / d), -127.0f), 127.0f));
        q3 = static_cast<int>(fminf(fmaxf(rintf(v.w / d), -127.0f), 127.0f));
    }
    int s = q0 + q1 + q2 + q3;
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    s += __shfl_xor(s, 4, 64);

    if (live) {
        codes[t] = (uint32_t(q0) & 0xFFu) | ((uint32_t(q1) & 0xFFu) << 8) |
                   ((uint32_t(q2) & 0xFFu) << 16) | ((uint32_t(q3) & 0xFFu) << 24);
        if (j == 0) {
            scales[blk] = d;
            sums[blk] = s;
        }
    }

    // ---- the fp6 section (every lane of the wave takes part in the shuffles)
    auto chunk = [](int a, int b, int c, int e, bool high) {
        auto dig = [high](int q) { return high ? e2m3_half_code(q >> 4) : e2m3_half_code(q & 15); };
        return dig(a) | (dig(b) << 6) | (dig(c) << 12) | (dig(e) << 18);
    };
    const uint32_t ch = chunk(q0, q1, q2, q3, true), cl = chunk(q0, q1, q2, q3, false);
    // dword k (lanes k = 0..5) of the 192-bit records: bits 32 k .. of lanes' 24-bit chunks
    const int p = j / 3, r = j % 3;
    const int src = 4 * p + r;
    const uint32_t h0 = __shfl(ch, src, 8), h1 = __shfl(ch, src + 1, 8);
    const uint32_t l0 = __shfl(cl, src, 8), l1 = __shfl(cl, src + 1, 8);
    if (in_k) {
        const int step = kb >> 1, u = kb & 1;
        uint32_t* slab = f6 + int64_t(step) * 32 * Mp;   // 128 Mp bytes per step
        const uint32_t dh = (h0 >> (8 * r)) | (h1 << (24 - 8 * r));
        const uint32_t dl = (l0 >> (8 * r)) | (l1 << (24 - 8 * r));
        const uint32_t hilo = bf16_hilo_bits(d);
        const uint32_t thilo = bf16_hilo_bits(product_f32(d, float(s)));
        auto put = [&](int uu, bool zero) {
            if (j < 4) {
                slab[((2 * uu) * Mp + m) * 4 + j] = zero ? 0u : dh;          // digits16, h
                slab[((2 * uu + 1) * Mp + m) * 4 + j] = zero ? 0u : dl;      // digits16, l
            } else if (j < 6) {
                slab[16 * Mp + ((2 * uu) * Mp + m) * 2 + (j - 4)] = zero ? 0u : dh;       // digits8, h
                slab[16 * Mp + ((2 * uu + 1) * Mp + m) * 2 + (j - 4)] = zero ? 0u : dl;   // digits8, l
            } else if (j == 6) {
                uint32_t* o = slab + 24 * Mp + (uu * Mp + m) * 2;                // outer
                o[0] = zero ? 0u : hilo;
                o[1] = zero ? 0u : hilo;
            } else {
                uint32_t* o = slab + 28 * Mp + (uu * Mp + m) * 2;                // min
                o[0] = zero ? 0u : ((thilo & 0xFFFFu) | (thilo << 16));
                o[1] = zero ? 0u : ((thilo >> 16) | (thilo & 0xFFFF0000u));
            }
        };
        put(u, false);
        if ((KB & 1) && kb == KB - 1) put(1, true);   // the step's second block does not exist
    }
}

hipError_t launch_quantize_act(const float* X, int8_t* codes, float* scales, int32_t* sums, uint8_t* f6, int64_t M,
                               int64_t K, hipStream_t s) {
    const int64_t Mp = f6_act_rows(M);
    const int KB = int(K / 32);
    const int block_groups = (KB + 3) / 4;
    const int64_t blocks = (Mp / 8) * block_groups;
    hipLaunchKernelGGL(quantize_act_kernel, dim3(unsigned(blocks)), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(X), reinterpret_cast<uint32_t*>(codes), scales,
                       sums, reinterpret_cast<uint32_t*>(f6), M, Mp, KB, block_groups);
    return hipGetLastError();
}

}  // namespace mq
