// mq_quantize_act kernel: f32 rows -> q8 blocks of 32 with an f32 scale.
//
// Per 32-value block ("minfer Architecture Execution Plan", C4 S2b design
// decision 4: amax, scale amax / 127, round half to even; the scale is kept in
// f32 here):  amax = max |x|;  d = amax / 127 (IEEE f32 division);
// q = clamp(rint(x / d), -127, 127) with a true division, q = 0 when d == 0;
// sum = sum of the 32 codes.
//
// Eight lanes own one block, four values each (one 16-byte load per lane), so
// a wave quantizes eight blocks and the block reductions are three DPP lane
// moves.  A wave takes the same block of eight consecutive rows, and a
// workgroup four consecutive blocks of those rows: each wave's stores of the
// row-major arrays below then fill whole 64- or 128-byte segments.  The kernel
// streams X once; at large sizes its vector instructions (about 240 per wave)
// take as long as its memory traffic, so addresses are a wave-uniform base plus
// a 32-bit lane offset and the fp6 digit codes are looked up four at a time.
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
    // workgroup: rows 8 rg .. 8 rg + 7 (of Mp) x blocks 4 bg .. 4 bg + 3; wave w: block 4 bg + w.
    // Every address is a base uniform over the wave (64-bit, scalar) plus a 32-bit lane offset.
    const int64_t rg = blockIdx.x / block_groups;
    const int bg = int(blockIdx.x % block_groups);
    const int j = int(threadIdx.x & 7);
    const int r = int((threadIdx.x >> 3) & 7);
    const int kb = 4 * bg + __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int64_t m0 = 8 * rg;
    const int64_t m = m0 + r;
    const bool in_k = kb < KB;        // uniform per wave
    const bool live = in_k && m < M;  // rows M..Mp-1 only get the fp6 section's zeros
    const int64_t blk0 = m0 * KB + kb;                       // block of the wave's first row
    const uint32_t row_q = __umul24(uint32_t(r), uint32_t(KB) * 8u) + uint32_t(j);   // this lane's quad past it
    const float4 v = live ? (X + blk0 * 8)[row_q] : make_float4(0.f, 0.f, 0.f, 0.f);

    float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    a = lanes8_max(a);
    const float d = a / 127.0f;

    int q0 = 0, q1 = 0, q2 = 0, q3 = 0;
    if (d > 0.0f) {
        q0 = static_cast<int>(fminf(fmaxf(rintf(v.x / d), -127.0f), 127.0f));
        q1 = static_cast<int>(fminf(fmaxf(rintf(v.y / d), -127.0f), 127.0f));
        q2 = static_cast<int>(fminf(fmaxf(rintf(v.z / d), -127.0f), 127.0f));
        q3 = static_cast<int>(fminf(fmaxf(rintf(v.w / d), -127.0f), 127.0f));
    }
    const int s = lanes8_sum(q0 + q1 + q2 + q3);

    const uint32_t w = (uint32_t(q0) & 0xFFu) | ((uint32_t(q1) & 0xFFu) << 8) | ((uint32_t(q2) & 0xFFu) << 16) |
                       ((uint32_t(q3) & 0xFFu) << 24);   // the four codes as bytes
    if (live) {
        (codes + blk0 * 8)[row_q] = w;
        if (j == 0) {
            const uint32_t row_b = __umul24(uint32_t(r), uint32_t(KB));
            (scales + blk0)[row_b] = d;
            (sums + blk0)[row_b] = s;
        }
    }

    // ---- the fp6 section (every lane of the wave takes part in the lane moves)
    // the 6-bit codes of the four values' digits, value i in bits 6 i .. 6 i + 5 (from one
    // code per byte); h = q >> 4 is the high nibble of q's byte read as signed, l its low one
    auto chunk = [](uint32_t c) {
        return (c & 0x3Fu) | ((c >> 2) & 0xFC0u) | ((c >> 4) & 0x3F000u) | ((c >> 6) & 0xFC0000u);
    };
    const uint32_t ch = chunk(e2m3_half_codes4<true>((w >> 4) & 0x0F0F0F0Fu));
    const uint32_t cl = chunk(e2m3_half_codes4<false>(w & 0x0F0F0F0Fu));
    // dword k (lanes k = 0..5) of the 192-bit records: bits 32 k .. of lanes' 24-bit chunks,
    // from the chunks of lanes 4 (k / 3) + k % 3 and the next one (k or k + 1, then k + 1
    // or k + 2: the same or the next two lanes, all in the lane's row of 16; DPP row
    // shifts, whose lanes that would read past the row are among those not stored)
    const int rr = j % 3;
    const bool second = j >= 3;
    const uint32_t ch1 = uint32_t(__builtin_amdgcn_mov_dpp(int(ch), 0x101, 0xF, 0xF, false));   // row_shl:1
    const uint32_t ch2 = uint32_t(__builtin_amdgcn_mov_dpp(int(ch), 0x102, 0xF, 0xF, false));   // row_shl:2
    const uint32_t cl1 = uint32_t(__builtin_amdgcn_mov_dpp(int(cl), 0x101, 0xF, 0xF, false));
    const uint32_t cl2 = uint32_t(__builtin_amdgcn_mov_dpp(int(cl), 0x102, 0xF, 0xF, false));
    const uint32_t h0 = second ? ch1 : ch, h1 = second ? ch2 : ch1;
    const uint32_t l0 = second ? cl1 : cl, l1 = second ? cl2 : cl1;
    if (in_k) {
        const int step = kb >> 1, u = kb & 1;
        uint32_t* slab = f6 + int64_t(step) * 32 * Mp;   // 128 Mp bytes per step
        const uint32_t dh = (h0 >> (8 * rr)) | (h1 << (24 - 8 * rr));
        const uint32_t dl = (l0 >> (8 * rr)) | (l1 << (24 - 8 * rr));
        const uint32_t hilo = bf16_hilo_bits(d);
        const uint32_t thilo = bf16_hilo_bits(product_f32(d, float(s)));
        // Two dword stores per lane: lanes 0..3 the digits16 records (h, then l), lanes 4, 5
        // the digits8 records, lane 6 the outer operand record and lane 7 the min operand
        // record (its two dwords).  Offsets in dwords past the slab, 32-bit (Mp <= 2^20).
        const uint32_t mp = uint32_t(Mp), mr = uint32_t(m0) + uint32_t(r);
        auto put = [&](int uu, bool zero) {
            const uint32_t uw = uint32_t(uu);
            uint32_t o1, o2, v1, v2;
            if (j < 4) {
                o1 = ((2 * uw) * mp + mr) * 4 + j;
                o2 = o1 + 4 * mp;
                v1 = dh;
                v2 = dl;
            } else if (j < 6) {
                o1 = 16 * mp + ((2 * uw) * mp + mr) * 2 + (j - 4);
                o2 = o1 + 2 * mp;
                v1 = dh;
                v2 = dl;
            } else {
                o1 = __umul24(j == 6 ? 24u : 28u, mp) + (uw * mp + mr) * 2;
                o2 = o1 + 1;
                v1 = j == 6 ? hilo : ((thilo & 0xFFFFu) | (thilo << 16));
                v2 = j == 6 ? hilo : ((thilo >> 16) | (thilo & 0xFFFF0000u));
            }
            slab[o1] = zero ? 0u : v1;
            slab[o2] = zero ? 0u : v2;
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
