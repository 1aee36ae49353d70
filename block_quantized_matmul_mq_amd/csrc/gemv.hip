// mq_gemv kernels: y = deq(W) x for one f32 activation row (the decode
// product of "minfer CUDA Backend Design", 4.4 Execution dispatch; here the
// activation stays f32 and is never quantized).
//
// Work split.  A row of K values is cut into K/32 "slices" of 32 values; the
// 64 lanes of a wave own 64 consecutive slices (one K-step of 2048 values) and
// a slice's 32 activation values stay in the lane's registers while the lane
// walks R weight rows, so each x value read from cache serves R rows.  KW
// waves of a workgroup share the same R rows and take every KW-th K-step;
// their partial sums meet in LDS.  Weight bytes are read once, with 16-byte
// (Q4_K) or dword (Q8_0, Q6_K: 34- and 210-byte blocks are only 2-byte
// aligned) loads; codes are unpacked in registers and scales applied per
// sub-block.  The product accumulates in f32.
//
// Per-type slice (s = slice index within the row):
//   Q4_K: super-block s/8, code chunk p = s%8 (16 bytes of qs at 16 + 16p):
//         low nibbles are values 64(p/2) + 16(p%2) + i, high nibbles the same
//         +32, i < 16; sub-blocks 2(p/2) and 2(p/2)+1.
//   Q6_K: super-block s/8, lane part p = s%8: values 128h + 32t + l for
//         h < 2, t < 4, l in [4p, 4p+4).
//   Q8_0: block s (32 consecutive values).
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

namespace {

struct SliceQ8_0 {
    float xv[32];
    float xsum;
    __device__ void load_x(const float* __restrict__ x, int s) {
        const float4* p = reinterpret_cast<const float4*>(x + 32 * s);
        xsum = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float4 v = p[i];
            xv[4 * i] = v.x; xv[4 * i + 1] = v.y; xv[4 * i + 2] = v.z; xv[4 * i + 3] = v.w;
            xsum += (v.x + v.y) + (v.z + v.w);
        }
    }
    // sum_i d * q_i * x_i with q_i = (byte_i ^ 0x80) - 128.
    __device__ float row_dot(const uint8_t* __restrict__ row, int s) const {
        const uint8_t* blk = row + 34 * s;
        const float d = half_bits_to_float(load_u16(blk));
        const uint8_t* cp = blk + 2;
        const uintptr_t a = reinterpret_cast<uintptr_t>(cp);
        const uint32_t* q = reinterpret_cast<const uint32_t*>(a & ~uintptr_t(3));
        uint32_t w[9];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = q[i];
        const bool odd = (a & 2) != 0;
        w[8] = odd ? q[8] : 0u;
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t c = odd ? align_byte(w[i + 1], w[i], 2) : w[i];
            c ^= 0x80808080u;
            dot = fmaf(ubyte_f<0>(c), xv[4 * i], dot);
            dot = fmaf(ubyte_f<1>(c), xv[4 * i + 1], dot);
            dot = fmaf(ubyte_f<2>(c), xv[4 * i + 2], dot);
            dot = fmaf(ubyte_f<3>(c), xv[4 * i + 3], dot);
        }
        return d * fmaf(-128.0f, xsum, dot);
    }
};

struct SliceQ4_K {
    float xlo[16], xhi[16];
    float slo, shi;
    int c, h;
    __device__ void load_x(const float* __restrict__ x, int s) {
        const int sb = s >> 3, p = s & 7;
        c = p >> 1;
        h = p & 1;
        const float* base = x + 256 * sb + 64 * c + 16 * h;
        slo = 0.f;
        shi = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 a = reinterpret_cast<const float4*>(base)[i];
            const float4 b = reinterpret_cast<const float4*>(base + 32)[i];
            xlo[4 * i] = a.x; xlo[4 * i + 1] = a.y; xlo[4 * i + 2] = a.z; xlo[4 * i + 3] = a.w;
            xhi[4 * i] = b.x; xhi[4 * i + 1] = b.y; xhi[4 * i + 2] = b.z; xhi[4 * i + 3] = b.w;
            slo += (a.x + a.y) + (a.z + a.w);
            shi += (b.x + b.y) + (b.z + b.w);
        }
    }
    __device__ float row_dot(const uint8_t* __restrict__ row, int s) const {
        const uint8_t* blk = row + 144 * (s >> 3);
        const uint4 hd = *reinterpret_cast<const uint4*>(blk);
        const uint4 qs = *reinterpret_cast<const uint4*>(blk + 16 + 16 * (s & 7));
        const float d = half_bits_to_float(hd.x & 0xFFFFu);
        const float dmin = half_bits_to_float(hd.x >> 16);
        uint32_t sc0, m0, sc1, m1;
        q4k_scale_min(hd.y, hd.z, hd.w, 2 * c, sc0, m0);
        q4k_scale_min(hd.y, hd.z, hd.w, 2 * c + 1, sc1, m1);
        const uint32_t qw[4] = {qs.x, qs.y, qs.z, qs.w};
        float dlo = 0.f, dhi = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = qw[i] & 0x0F0F0F0Fu;
            const uint32_t hi = (qw[i] >> 4) & 0x0F0F0F0Fu;
            dlo = fmaf(ubyte_f<0>(lo), xlo[4 * i], dlo);
            dlo = fmaf(ubyte_f<1>(lo), xlo[4 * i + 1], dlo);
            dlo = fmaf(ubyte_f<2>(lo), xlo[4 * i + 2], dlo);
            dlo = fmaf(ubyte_f<3>(lo), xlo[4 * i + 3], dlo);
            dhi = fmaf(ubyte_f<0>(hi), xhi[4 * i], dhi);
            dhi = fmaf(ubyte_f<1>(hi), xhi[4 * i + 1], dhi);
            dhi = fmaf(ubyte_f<2>(hi), xhi[4 * i + 2], dhi);
            dhi = fmaf(ubyte_f<3>(hi), xhi[4 * i + 3], dhi);
        }
        const float scaled = fmaf(float(sc0), dlo, float(sc1) * dhi);
        const float mins = fmaf(float(m0), slo, float(m1) * shi);
        return fmaf(d, scaled, -dmin * mins);
    }
};

struct SliceQ6_K {
    float xv[2][4][4];  // [h][t][k]: value 128h + 32t + 4p + k
    float xs[2][4];
    int p;
    __device__ void load_x(const float* __restrict__ x, int s) {
        const int sb = s >> 3;
        p = s & 7;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const float4 v = *reinterpret_cast<const float4*>(x + 256 * sb + 128 * h + 32 * t + 4 * p);
                xv[h][t][0] = v.x; xv[h][t][1] = v.y; xv[h][t][2] = v.z; xv[h][t][3] = v.w;
                xs[h][t] = (v.x + v.y) + (v.z + v.w);
            }
    }
    __device__ float row_dot(const uint8_t* __restrict__ row, int s) const {
        const uint8_t* blk = row + 210 * (s >> 3);
        const float d = half_bits_to_float(load_u16(blk + 208));
        const int u = p >> 2;  // which of the two 16-value halves of each 32-run
        float acc = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t ql0 = load_u32_a2(blk + 64 * h + 4 * p);
            const uint32_t ql1 = load_u32_a2(blk + 64 * h + 32 + 4 * p);
            const uint32_t qh = load_u32_a2(blk + 128 + 32 * h + 4 * p);
            const uint32_t sc_lo = load_u32_a2(blk + 192 + 8 * h);      // scales 8h .. 8h+3
            const uint32_t sc_hi = load_u32_a2(blk + 192 + 8 * h + 4);  // scales 8h+4 .. 8h+7
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const uint32_t src = (t & 1) ? ql1 : ql0;
                const uint32_t low = (t < 2 ? src : (src >> 4)) & 0x0F0F0F0Fu;
                const uint32_t high = (qh >> (2 * t)) & 0x03030303u;
                const uint32_t code = low | (high << 4);
                float dot = ubyte_f<0>(code) * xv[h][t][0];
                dot = fmaf(ubyte_f<1>(code), xv[h][t][1], dot);
                dot = fmaf(ubyte_f<2>(code), xv[h][t][2], dot);
                dot = fmaf(ubyte_f<3>(code), xv[h][t][3], dot);
                dot = fmaf(-32.0f, xs[h][t], dot);
                // signed sub-scale 8h + 2t + u
                const int g = 2 * t + u;
                const uint32_t word = g < 4 ? sc_lo : sc_hi;
                const float sc = float(int32_t(word << (24 - 8 * (g & 3))) >> 24);
                acc = fmaf(sc, dot, acc);
            }
        }
        return d * acc;
    }
};

template <int QT> struct SliceOf;
template <> struct SliceOf<kQ8_0> { using T = SliceQ8_0; };
template <> struct SliceOf<kQ4_K> { using T = SliceQ4_K; };
template <> struct SliceOf<kQ6_K> { using T = SliceQ6_K; };

template <int QT, int R, int KW>
__global__ __launch_bounds__(64 * KW) void gemv_kernel(const uint8_t* __restrict__ W,
                                                       const float* __restrict__ x,
                                                       float* __restrict__ y, int N, int K,
                                                       int64_t row_bytes) {
    using Slice = typename SliceOf<QT>::T;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row0 = blockIdx.x * R;
    const int nslices = K >> 5;

    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;

    for (int step = wave; step * 64 < nslices; step += KW) {
        const int s = step * 64 + lane;
        if (s < nslices) {
            Slice sl;
            sl.load_x(x, s);
#pragma unroll
            for (int r = 0; r < R; ++r) {
                if (row0 + r < N) acc[r] += sl.row_dot(W + int64_t(row0 + r) * row_bytes, s);
            }
        }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = wave_sum(acc[r]);

    if constexpr (KW == 1) {
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                if (row0 + r < N) y[row0 + r] = acc[r];
        }
    } else {
        __shared__ float part[KW][R];
        if (lane == 0) {
#pragma unroll
            for (int r = 0; r < R; ++r) part[wave][r] = acc[r];
        }
        __syncthreads();
        if (threadIdx.x < R && row0 + int(threadIdx.x) < N) {
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < KW; ++w) v += part[w][threadIdx.x];
            y[row0 + threadIdx.x] = v;
        }
    }
}

template <int QT, int R, int KW>
hipError_t launch_one(const uint8_t* W, const float* x, float* y, int64_t N, int64_t K, int64_t row_bytes,
                      hipStream_t s) {
    const int64_t blocks = (N + R - 1) / R;
    hipLaunchKernelGGL((gemv_kernel<QT, R, KW>), dim3(unsigned(blocks)), dim3(64 * KW), 0, s, W, x, y,
                       int(N), int(K), row_bytes);
    return hipGetLastError();
}

template <int QT>
hipError_t launch_typed(const uint8_t* W, const float* x, float* y, int64_t N, int64_t K,
                        int64_t row_bytes, hipStream_t s, const char** name) {
    const int64_t steps = (K / 32 + 63) / 64;
    if (steps >= 4) {
        if (N >= 8192) { *name = "gemv<R4,KW4>"; return launch_one<QT, 4, 4>(W, x, y, N, K, row_bytes, s); }
        *name = "gemv<R2,KW4>";
        return launch_one<QT, 2, 4>(W, x, y, N, K, row_bytes, s);
    }
    if (steps >= 2) {
        if (N >= 8192) { *name = "gemv<R4,KW2>"; return launch_one<QT, 4, 2>(W, x, y, N, K, row_bytes, s); }
        *name = "gemv<R2,KW2>";
        return launch_one<QT, 2, 2>(W, x, y, N, K, row_bytes, s);
    }
    if (N >= 8192) { *name = "gemv<R4,KW1>"; return launch_one<QT, 4, 1>(W, x, y, N, K, row_bytes, s); }
    *name = "gemv<R2,KW1>";
    return launch_one<QT, 2, 1>(W, x, y, N, K, row_bytes, s);
}

}  // namespace

hipError_t launch_gemv(int type, const uint8_t* W, const float* x, float* y, int64_t N, int64_t K,
                       hipStream_t s, const char** name) {
    switch (type) {
        case kQ8_0: return launch_typed<kQ8_0>(W, x, y, N, K, (K / 32) * 34, s, name);
        case kQ4_K: return launch_typed<kQ4_K>(W, x, y, N, K, (K / 256) * 144, s, name);
        case kQ6_K: return launch_typed<kQ6_K>(W, x, y, N, K, (K / 256) * 210, s, name);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mq
