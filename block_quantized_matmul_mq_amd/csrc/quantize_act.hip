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
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

__global__ __launch_bounds__(256) void quantize_act_kernel(const float4* __restrict__ X,
                                                           uint32_t* __restrict__ codes,
                                                           float* __restrict__ scales,
                                                           int32_t* __restrict__ sums,
                                                           int64_t n_quads) {
    const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const bool live = t < n_quads;
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
    }
}

hipError_t launch_quantize_act(const float* X, int8_t* codes, float* scales, int32_t* sums,
                               int64_t M, int64_t K, hipStream_t s) {
    const int64_t n_quads = M * K / 4;
    const int64_t blocks = (n_quads + 255) / 256;
    hipLaunchKernelGGL(quantize_act_kernel, dim3(unsigned(blocks)), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(X), reinterpret_cast<uint32_t*>(codes), scales,
                       sums, n_quads);
    return hipGetLastError();
}

}  // namespace mq
