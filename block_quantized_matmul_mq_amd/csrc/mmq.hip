// mq_gemm kernels: the int8 "MMQ" prefill product ("minfer CUDA Backend
// Design", 4.4 Execution dispatch: prefill multiplies the weights' block codes
// with an activation plane quantized to q8 blocks on int8 matrix units).
//
//   Y[m][n] = sum_b dx[m][b] * ( dw[n][b] * D[m][n][b] - mw[n][b] * S[m][b] )
//
// D are exact int32 dot products of weight codes with activation codes per
// 32-value block (per 16-value group for Q6_K, whose sub-scales change every 16
// values); dx/S are the activation block scale and code sum; dw (and mw, the
// Q4_K min term) are the weight's per-block factors.
//
// Tiling.  A 256-thread workgroup (4 waves, 2 x 2) owns a 128 x 128 tile of Y
// and walks K in steps of 128 values (4 blocks).  Each step stages the int8
// activation codes and the weight codes -- unpacked from the raw block bytes
// into int8 (Q4_K 0..15, Q6_K code-32, Q8_0 q) -- into LDS with the per-block
// factors, then every wave runs v_mfma_i32_32x32x32_i8 (v_mfma_i32_32x32x16_i8
// per 16-value half for Q6_K) on its 2 x 2 sub-tiles of 32 x 32 and applies the
// block factors to the fresh int32 dots in f32.  LDS rows are padded by 16
// bytes so the 16-byte fragment reads of 32 consecutive rows hit distinct banks.
//
// Workgroups are numbered so that the ones sharing a weight tile run on the
// same XCD (consecutive workgroup ids are dealt round-robin to the 8 XCDs, each
// with its own L2): the weight tile then comes from HBM once per XCD.
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int KS = 128;        // K values per step
constexpr int NB = KS / 32;    // 32-blocks per step
constexpr int LDA = KS + 16;   // padded LDS row (bytes)
constexpr int kXcds = 8;

template <int QT> struct Groups { static constexpr int per_step = NB; };
template <> struct Groups<kQ6_K> { static constexpr int per_step = 2 * NB; };

// Row index (within a 32-row MFMA tile) of accumulator element v for lane group g = lane / 32.
__device__ __forceinline__ int acc_row(int v, int g) { return 8 * (v >> 2) + 4 * g + (v & 3); }

template <int QT>
__device__ __forceinline__ void stage_weights(const uint8_t* __restrict__ W, int64_t row_bytes, int n0,
                                              int N, int k0, int K, int8_t* Bs, float (*dws)[BN],
                                              float (*mws)[BN]) {
    const int t = threadIdx.x;
    if constexpr (QT == kQ4_K) {
        // 128 rows x 4 code chunks of 16 bytes (half a super-block per step).
        const int sb = k0 >> 8;
        const int half = (k0 >> 7) & 1;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int u = t + 256 * it;
            const int row = u >> 2;
            const int pp = u & 3;
            const int p = 4 * half + pp;        // chunk within the super-block
            const int c = p >> 1, h = p & 1;
            const int n = n0 + row;
            uint4 q = make_uint4(0, 0, 0, 0);
            const uint8_t* blk = W + int64_t(n) * row_bytes + 144 * sb;
            if (n < N) q = *reinterpret_cast<const uint4*>(blk + 16 + 16 * p);
            const uint4 lo = make_uint4(q.x & 0x0F0F0F0Fu, q.y & 0x0F0F0F0Fu, q.z & 0x0F0F0F0Fu,
                                        q.w & 0x0F0F0F0Fu);
            const uint4 hi = make_uint4((q.x >> 4) & 0x0F0F0F0Fu, (q.y >> 4) & 0x0F0F0F0Fu,
                                        (q.z >> 4) & 0x0F0F0F0Fu, (q.w >> 4) & 0x0F0F0F0Fu);
            const int pos = 64 * c + 16 * h - 128 * half;  // value offset within this step
            *reinterpret_cast<uint4*>(Bs + row * LDA + pos) = lo;
            *reinterpret_cast<uint4*>(Bs + row * LDA + pos + 32) = hi;
            if (h == 0) {
                float ws0 = 0.f, ws1 = 0.f, wm0 = 0.f, wm1 = 0.f;
                if (n < N) {
                    const uint4 hd = *reinterpret_cast<const uint4*>(blk);
                    const float d = half_bits_to_float(hd.x & 0xFFFFu);
                    const float dmin = half_bits_to_float(hd.x >> 16);
                    uint32_t sc, mn;
                    q4k_scale_min(hd.y, hd.z, hd.w, 2 * c, sc, mn);
                    ws0 = d * float(sc);
                    wm0 = dmin * float(mn);
                    q4k_scale_min(hd.y, hd.z, hd.w, 2 * c + 1, sc, mn);
                    ws1 = d * float(sc);
                    wm1 = dmin * float(mn);
                }
                const int jb = 2 * c - 4 * half;  // local block index of sub-block 2c
                dws[jb][row] = ws0;
                dws[jb + 1][row] = ws1;
                mws[jb][row] = wm0;
                mws[jb + 1][row] = wm1;
            }
        }
    } else if constexpr (QT == kQ8_0) {
        // 128 rows x 4 blocks of 34 bytes (2-byte aligned): aligned dwords, realigned.
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int u = t + 256 * it;
            const int row = u >> 2;
            const int bi = u & 3;
            const int kb = (k0 >> 5) + bi;
            const int n = n0 + row;
            uint32_t c[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            float d = 0.f;
            if (n < N && kb < (K >> 5)) {
                const uint8_t* blk = W + int64_t(n) * row_bytes + 34 * int64_t(kb);
                d = half_bits_to_float(load_u16(blk));
                const uintptr_t a = reinterpret_cast<uintptr_t>(blk + 2);
                const uint32_t* q = reinterpret_cast<const uint32_t*>(a & ~uintptr_t(3));
                uint32_t w[9];
#pragma unroll
                for (int i = 0; i < 8; ++i) w[i] = q[i];
                const bool odd = (a & 2) != 0;
                w[8] = 0;
                if (odd) w[8] = q[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) c[i] = odd ? align_byte(w[i + 1], w[i], 2) : w[i];
            }
            *reinterpret_cast<uint4*>(Bs + row * LDA + 32 * bi) = make_uint4(c[0], c[1], c[2], c[3]);
            *reinterpret_cast<uint4*>(Bs + row * LDA + 32 * bi + 16) = make_uint4(c[4], c[5], c[6], c[7]);
            dws[bi][row] = d;
        }
    } else {
        // Q6_K: half h of a 210-byte super-block per step; part p owns values
        // 128h + 32t + l, l in [4p, 4p+4), t < 4.
        const int sb = k0 >> 8;
        const int h = (k0 >> 7) & 1;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int u = t + 256 * it;
            const int row = u >> 3;
            const int p = u & 7;
            const int n = n0 + row;
            uint32_t ql0 = 0, ql1 = 0, qh = 0;
            const uint8_t* blk = W + int64_t(n) * row_bytes + 210 * sb;
            if (n < N) {
                ql0 = load_u32_a2(blk + 64 * h + 4 * p);
                ql1 = load_u32_a2(blk + 64 * h + 32 + 4 * p);
                qh = load_u32_a2(blk + 128 + 32 * h + 4 * p);
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const uint32_t src = (tt & 1) ? ql1 : ql0;
                const uint32_t low = (tt < 2 ? src : (src >> 4)) & 0x0F0F0F0Fu;
                const uint32_t high = (qh >> (2 * tt)) & 0x03030303u;
                uint32_t code = low | (high << 4);
                // per byte: code - 32 as int8 ((c + 128) - 32, then flip the sign bit back)
                code = ((code | 0x80808080u) - 0x20202020u) ^ 0x80808080u;
                if (n >= N) code = 0;
                *reinterpret_cast<uint32_t*>(Bs + row * LDA + 32 * tt + 4 * p) = code;
            }
            if (p == 0) {
                float d = 0.f;
                uint32_t s0 = 0, s1 = 0;
                if (n < N) {
                    d = half_bits_to_float(load_u16(blk + 208));
                    s0 = load_u32_a2(blk + 192 + 8 * h);
                    s1 = load_u32_a2(blk + 192 + 8 * h + 4);
                }
#pragma unroll
                for (int g = 0; g < 8; ++g) {
                    const uint32_t word = g < 4 ? s0 : s1;
                    const float sc = float(int32_t(word << (24 - 8 * (g & 3))) >> 24);
                    dws[g][row] = d * sc;
                }
            }
        }
    }
}

template <int QT, bool DUMP>
__global__ __launch_bounds__(256) void mmq_kernel(const uint8_t* __restrict__ W,
                                                  const int8_t* __restrict__ codes,
                                                  const float* __restrict__ xscale,
                                                  const int32_t* __restrict__ xsum,
                                                  float* __restrict__ Y, int32_t* __restrict__ dots,
                                                  int M, int N, int K, int64_t row_bytes,
                                                  int tiles_m, int tiles_total) {
    constexpr int NG = Groups<QT>::per_step;
    __shared__ __attribute__((aligned(16))) int8_t As[BM * LDA];
    __shared__ __attribute__((aligned(16))) int8_t Bs[BN * LDA];
    __shared__ __attribute__((aligned(16))) float dxs[NB][BM];
    __shared__ __attribute__((aligned(16))) float txs[NB][BM];
    __shared__ float dws[NG][BN];
    __shared__ float mws[NB][BN];

    // XCD-aware tile order: workgroups that land on one XCD take consecutive logical tiles.
    int bid = blockIdx.x;
    int logical = bid;
    if (tiles_total % kXcds == 0) logical = (bid % kXcds) * (tiles_total / kXcds) + bid / kXcds;
    const int tm = logical % tiles_m;
    const int tn = logical / tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int g = lane >> 5;   // lane group: which half of each 32-value block this lane feeds
    const int r32 = lane & 31;
    const int KB = K >> 5;

    float acc[2][2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    for (int k0 = 0; k0 < K; k0 += KS) {
        __syncthreads();
        // activation codes: 128 rows x 128 bytes, 4 x 16 bytes per thread
        {
            const int row = t >> 1, half = t & 1;
            const int m = m0 + row;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = half * 64 + 16 * i;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (m < M && k0 + kk < K)
                    v = *reinterpret_cast<const uint4*>(codes + int64_t(m) * K + k0 + kk);
                *reinterpret_cast<uint4*>(As + row * LDA + kk) = v;
            }
        }
        if (t < BM) {
            const int m = m0 + t;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int kb = (k0 >> 5) + b;
                float dx = 0.f, tx = 0.f;
                if (m < M && kb < KB) {
                    dx = xscale[int64_t(m) * KB + kb];
                    if constexpr (QT == kQ4_K) tx = dx * float(xsum[int64_t(m) * KB + kb]);
                }
                dxs[b][t] = dx;
                txs[b][t] = tx;
            }
        }
        stage_weights<QT>(W, row_bytes, n0, N, k0, K, Bs, dws, mws);
        __syncthreads();

#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int kb = (k0 >> 5) + b;
            if constexpr (QT == kQ6_K) {
                long a_lo[2], a_hi[2], b_lo[2], b_hi[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int8_t* ap = As + (64 * wm + 32 * i + r32) * LDA + 32 * b + 8 * g;
                    a_lo[i] = *reinterpret_cast<const long*>(ap);
                    a_hi[i] = *reinterpret_cast<const long*>(ap + 16);
                    const int8_t* bp = Bs + (64 * wn + 32 * i + r32) * LDA + 32 * b + 8 * g;
                    b_lo[i] = *reinterpret_cast<const long*>(bp);
                    b_hi[i] = *reinterpret_cast<const long*>(bp + 16);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int n = 64 * wn + 32 * j + r32;
                    const float s_lo = dws[2 * b][n], s_hi = dws[2 * b + 1][n];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        v16i z = {};
                        const v16i dlo = __builtin_amdgcn_mfma_i32_32x32x16_i8(a_lo[i], b_lo[j], z, 0, 0, 0);
                        const v16i dhi = __builtin_amdgcn_mfma_i32_32x32x16_i8(a_hi[i], b_hi[j], z, 0, 0, 0);
                        const int mb = 64 * wm + 32 * i;
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const float4 dx4 = *reinterpret_cast<const float4*>(&dxs[b][mb + 8 * q4 + 4 * g]);
                            const float dxv[4] = {dx4.x, dx4.y, dx4.z, dx4.w};
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int v = 4 * q4 + e;
                                const float w = fmaf(float(dlo[v]), s_lo, float(dhi[v]) * s_hi);
                                acc[i][j][v] = fmaf(dxv[e], w, acc[i][j][v]);
                                if constexpr (DUMP) {
                                    const int m = m0 + mb + acc_row(v, g);
                                    const int nn = n0 + n;
                                    if (m < M && nn < N && kb < KB) {
                                        const int64_t o = (int64_t(m) * N + nn) * (2 * KB) + 2 * kb;
                                        dots[o] = dlo[v];
                                        dots[o + 1] = dhi[v];
                                    }
                                }
                            }
                        }
                    }
                }
            } else {
                v4i af[2], bf[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    af[i] = *reinterpret_cast<const v4i*>(As + (64 * wm + 32 * i + r32) * LDA + 32 * b + 16 * g);
                    bf[i] = *reinterpret_cast<const v4i*>(Bs + (64 * wn + 32 * i + r32) * LDA + 32 * b + 16 * g);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int n = 64 * wn + 32 * j + r32;
                    const float wsc = dws[b][n];
                    float wmn = 0.f;
                    if constexpr (QT == kQ4_K) wmn = mws[b][n];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        v16i z = {};
                        const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], z, 0, 0, 0);
                        const int mb = 64 * wm + 32 * i;
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            const float4 dx4 = *reinterpret_cast<const float4*>(&dxs[b][mb + 8 * q4 + 4 * g]);
                            const float dxv[4] = {dx4.x, dx4.y, dx4.z, dx4.w};
                            float txv[4] = {0.f, 0.f, 0.f, 0.f};
                            if constexpr (QT == kQ4_K) {
                                const float4 t4 = *reinterpret_cast<const float4*>(&txs[b][mb + 8 * q4 + 4 * g]);
                                txv[0] = t4.x; txv[1] = t4.y; txv[2] = t4.z; txv[3] = t4.w;
                            }
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                const int v = 4 * q4 + e;
                                float a = fmaf(float(D[v]), dxv[e] * wsc, acc[i][j][v]);
                                if constexpr (QT == kQ4_K) a = fmaf(-txv[e], wmn, a);
                                acc[i][j][v] = a;
                                if constexpr (DUMP) {
                                    const int m = m0 + mb + acc_row(v, g);
                                    const int nn = n0 + n;
                                    if (m < M && nn < N && kb < KB) dots[(int64_t(m) * N + nn) * KB + kb] = D[v];
                                }
                            }
                        }
                    }
                }
            }
        }
    }

    // Y store: for a fixed accumulator element the 32 lanes of a group write 32 consecutive n.
    // The block-dot export variant stores only the dots.
    if constexpr (DUMP) return;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + 64 * wn + 32 * j + r32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + 64 * wm + 32 * i + acc_row(v, g);
                if (m < M && n < N) Y[int64_t(m) * N + n] = acc[i][j][v];
            }
        }
}

template <int QT>
hipError_t launch_typed(const uint8_t* W, const int8_t* codes, const float* xs, const int32_t* xsum,
                        float* Y, int32_t* dots, int64_t M, int64_t N, int64_t K, int64_t row_bytes,
                        hipStream_t s) {
    const int tiles_m = int((M + BM - 1) / BM);
    const int tiles_n = int((N + BN - 1) / BN);
    const int total = tiles_m * tiles_n;
    if (dots) {
        hipLaunchKernelGGL((mmq_kernel<QT, true>), dim3(total), dim3(256), 0, s, W, codes, xs, xsum, Y, dots,
                           int(M), int(N), int(K), row_bytes, tiles_m, total);
    } else {
        hipLaunchKernelGGL((mmq_kernel<QT, false>), dim3(total), dim3(256), 0, s, W, codes, xs, xsum, Y,
                           dots, int(M), int(N), int(K), row_bytes, tiles_m, total);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mmq(int type, const uint8_t* W, const int8_t* codes, const float* xs, const int32_t* xsum,
                      float* Y, int32_t* dots, int64_t M, int64_t N, int64_t K, hipStream_t s,
                      const char** name) {
    switch (type) {
        case kQ8_0:
            *name = "mmq<q8_0>";
            return launch_typed<kQ8_0>(W, codes, xs, xsum, Y, dots, M, N, K, (K / 32) * 34, s);
        case kQ4_K:
            *name = "mmq<q4_K>";
            return launch_typed<kQ4_K>(W, codes, xs, xsum, Y, dots, M, N, K, (K / 256) * 144, s);
        case kQ6_K:
            *name = "mmq<q6_K>";
            return launch_typed<kQ6_K>(W, codes, xs, xsum, Y, dots, M, N, K, (K / 256) * 210, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mq
