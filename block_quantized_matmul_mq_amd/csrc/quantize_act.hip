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
// shuffles.  The kernel streams X once: it is HBM-bound.
//
// It also writes the operand plane of the fp8 matrix-unit product, per 64-value step t
// (two blocks) of each row: a 128-byte digit record and a 16-byte scale record.  Each
// code is written as two exact fp8 (OCP e4m3) digit bytes: |q| = 16 h + l with h in
// [0, 7], l in [0, 15], both digits carrying the sign of q.  The l byte is the sign bit
// over l itself: e4m3 bytes 0..15 encode exactly l * 2^-9 (subnormals and the first
// binade share the spacing 2^-9).  The h byte encodes 16 h * 2^-9 = h * 2^-5 (a normal
// number).  Block b = 2t + u of the row takes bytes 64u.. of the digit record as
// [h of its values 0..31 | l of its values 0..31]: each 32-byte half meets the block's 32
// weight codes, sum_j 16 h_j c_j + sum_j l_j c_j = sum_j q_j c_j.  The scale record is
// (scale of block 2t, scale of block 2t + 1, code sum of 2t, code sum of 2t + 1).  A step
// of K that holds only one block (K % 64 == 32) has zero digits, scale and sum in the
// second half.
//
// And the fp6 section of the plane (the operands of the fp6 matrix-unit product; layout in
// mq_internal.h): each code as q = 16 h + l with h = q >> 4 in [-8, 7] and l = q & 15, as
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

// e4m3 bytes of the digits of a code q in [-127, 127] (see above).
__device__ __forceinline__ uint32_t fp8_digit_l(int q) {
    return (uint32_t(q < 0) << 7) | (uint32_t(abs(q)) & 15u);
}
__device__ __forceinline__ uint32_t fp8_digit_h(int q) {
    // h * 2^-5 for h = 0..7: 0, 2^-5, 2^-4, 1.5 2^-4, 2^-3, 1.25 2^-3, 1.5 2^-3, 1.75 2^-3
    constexpr uint64_t kTable = 0x262422201C181000ull;
    const uint32_t h = uint32_t(abs(q)) >> 4;
    return (uint32_t(q < 0) << 7) | uint32_t((kTable >> (8 * h)) & 0xFFu);
}

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
                                                           uint32_t* __restrict__ digits,
                                                           uint32_t* __restrict__ step_scales,
                                                           uint32_t* __restrict__ f6, int64_t M, int64_t Mp,
                                                           int KB, int64_t n_quads, int64_t n_quads_padded) {
    const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const bool live = t < n_quads;   // rows 0..M-1; t < n_quads_padded covers the fp6 padding rows
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
        if ((t & 7) == 0) {
            scales[t >> 3] = d;
            sums[t >> 3] = s;
        }
        // lane j = t % 8 of the block holds values 4j..4j+3: bytes 4j.. of the h half and
        // of the l half of the block's 64 bytes in the row's digit record of step kb / 2
        const uint32_t hb = fp8_digit_h(q0) | (fp8_digit_h(q1) << 8) | (fp8_digit_h(q2) << 16) | (fp8_digit_h(q3) << 24);
        const uint32_t lb = fp8_digit_l(q0) | (fp8_digit_l(q1) << 8) | (fp8_digit_l(q2) << 16) | (fp8_digit_l(q3) << 24);
        const int64_t blk = t >> 3;
        const int64_t m = blk / KB;
        const int kb = int(blk % KB);
        const int T = (KB + 1) >> 1;
        const int j = int(t & 7);
        uint32_t* rec = digits + (m * T + (kb >> 1)) * 32 + 16 * (kb & 1) + j;
        rec[0] = hb;
        rec[8] = lb;
        uint32_t* srec = step_scales + (int64_t(kb >> 1) * M + m) * 4;
        if (j == 0) {
            srec[kb & 1] = __float_as_uint(d);
            srec[2 + (kb & 1)] = uint32_t(s);
        }
        if ((KB & 1) && kb == KB - 1) {   // the step's second block does not exist: zeros
            rec[16] = 0u;
            rec[24] = 0u;
            if (j == 0) srec[1] = srec[3] = 0u;
        }
    }

    // ---- the fp6 section (every lane of the wave takes part in the shuffles)
    const int j = int(threadIdx.x & 7);
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
    if (t < n_quads_padded) {
        const int64_t blk = t >> 3;
        const int64_t m = blk / KB;
        const int kb = int(blk % KB);
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

hipError_t launch_quantize_act(const float* X, int8_t* codes, float* scales, int32_t* sums, uint8_t* digits,
                               uint8_t* step_scales, uint8_t* f6, int64_t M, int64_t K, hipStream_t s) {
    const int64_t Mp = f6_act_rows(M);
    const int64_t n_quads = M * K / 4, n_quads_padded = Mp * K / 4;
    const int64_t blocks = (n_quads_padded + 255) / 256;
    hipLaunchKernelGGL(quantize_act_kernel, dim3(unsigned(blocks)), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(X), reinterpret_cast<uint32_t*>(codes), scales,
                       sums, reinterpret_cast<uint32_t*>(digits), reinterpret_cast<uint32_t*>(step_scales),
                       reinterpret_cast<uint32_t*>(f6), M, Mp, int(K / 32), n_quads, n_quads_padded);
    return hipGetLastError();
}

}  // namespace mq
