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
// and walks K in steps of 128 values (4 blocks); each wave owns 2 x 2 MFMA
// tiles of 32 x 32.  The global data of step s+1 (activation codes, raw weight
// bytes, block factors) is loaded into registers while step s computes from
// LDS; between steps the registers are unpacked into LDS (weight codes become
// int8: Q4_K 0..15, Q6_K code-32, Q8_0 q).  LDS rows are padded by 16 bytes so
// the 16-byte fragment reads of 32 consecutive rows hit distinct banks.
//
// Per block and 32 x 32 tile the work is split between the matrix unit and the
// vector ALU so that the vector ALU does two operations per output element and
// block (convert, fused multiply-add):
//   * v_mfma_i32_32x32x32_i8 forms the exact block dots D
//     (v_mfma_i32_32x32x16_i8 per 16-value group for Q6_K);
//   * v_mfma_f32_32x32x1_2b_f32 forms the two outer products dx (x) dw of a pair
//     of blocks: the f32 scale of every element of both blocks;
//   * the vector ALU accumulates acc += float(D) * scale;
//   * for Q4_K the min term sum_b (dx S)[m][b] * mw[n][b] is a small GEMM over
//     blocks, accumulated straight into acc by v_mfma_f32_32x32x2_f32.
// Workgroups are numbered so that the ones sharing a weight tile run on the
// same XCD (consecutive workgroup ids are dealt round-robin to the 8 XCDs, each
// with its own L2): a weight tile then comes from HBM once per XCD.
#include <algorithm>

#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int KS = 128;        // K values per step
constexpr int NB = KS / 32;    // 32-blocks per step
constexpr int LDA = KS + 16;   // padded LDS row (bytes)
constexpr int kXcds = 8;
constexpr int kTargetWorkgroups = 512;   // two resident 256-thread workgroups on each of 256 CUs
constexpr int kMinStepsPerSplit = 2;

template <int QT> struct Groups { static constexpr int per_step = NB; };
template <> struct Groups<kQ6_K> { static constexpr int per_step = 2 * NB; };

// Row index (within a 32-row MFMA tile) of accumulator element v for lane group g = lane / 32.
__device__ __forceinline__ int acc_row(int v, int g) { return 8 * (v >> 2) + 4 * g + (v & 3); }

// ------------------------------------------------------------------ staging
// Raw global data of one K-step, held in registers from the load (issued
// before the previous step's compute) to the LDS write after it.  Rows past N
// (M) re-read row N-1 (M-1): their outputs are never stored.
template <int QT> struct WeightRegs;

template <> struct WeightRegs<kQ4_K> {
    // Thread t owns pieces u = t and t + 256: row u/4, 16-byte code chunk 4*half + u%4
    // of the super-block (half = which 128 values of it this step covers), and the
    // 16-byte header (d, dmin, packed scales) of that row's super-block.
    uint4 q[2], hd[2];
    __device__ void load(const uint8_t* W, int64_t rb, int n0, int N, int k0, int) {
        const int t = threadIdx.x, sb = k0 >> 8, half = (k0 >> 7) & 1;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int u = t + 256 * it, row = u >> 2, p = 4 * half + (u & 3);
            const int n = min(n0 + row, N - 1);
            const uint8_t* blk = W + int64_t(n) * rb + 144 * sb;
            q[it] = *reinterpret_cast<const uint4*>(blk + 16 + 16 * p);
            hd[it] = *reinterpret_cast<const uint4*>(blk);
        }
    }
    __device__ void store(int8_t* Bs, float (*dws)[BN], float (*mws)[BN], int k0) const {
        const int t = threadIdx.x, half = (k0 >> 7) & 1;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int u = t + 256 * it, row = u >> 2, p = 4 * half + (u & 3);
            const int c = p >> 1, h = p & 1;
            const uint4 v = q[it];
            const uint4 lo = make_uint4(v.x & 0x0F0F0F0Fu, v.y & 0x0F0F0F0Fu, v.z & 0x0F0F0F0Fu, v.w & 0x0F0F0F0Fu);
            const uint4 hi = make_uint4((v.x >> 4) & 0x0F0F0F0Fu, (v.y >> 4) & 0x0F0F0F0Fu,
                                        (v.z >> 4) & 0x0F0F0F0Fu, (v.w >> 4) & 0x0F0F0F0Fu);
            // chunk c holds values 64c..64c+63: low nibbles the first 32, high nibbles the next 32
            const int pos = 64 * c + 16 * h - 128 * half;   // value offset within this step
            *reinterpret_cast<uint4*>(Bs + row * LDA + pos) = lo;
            *reinterpret_cast<uint4*>(Bs + row * LDA + pos + 32) = hi;
            if (h == 0) {
                const float d = half_bits_to_float(hd[it].x & 0xFFFFu);
                const float dmin = half_bits_to_float(hd[it].x >> 16);
                const int jb = 2 * c - 4 * half;   // step-local block of sub-block 2c
                uint32_t sc, mn;
                q4k_scale_min(hd[it].y, hd[it].z, hd[it].w, 2 * c, sc, mn);
                dws[jb][row] = d * float(sc);
                mws[jb][row] = -(dmin * float(mn));
                q4k_scale_min(hd[it].y, hd[it].z, hd[it].w, 2 * c + 1, sc, mn);
                dws[jb + 1][row] = d * float(sc);
                mws[jb + 1][row] = -(dmin * float(mn));
            }
        }
    }
};

template <> struct WeightRegs<kQ8_0> {
    // Thread t owns pieces u = t and t + 256: block u%4 of this step in row u/4, read as
    // the 9 naturally aligned dwords that cover its 34 bytes (every one of them holds
    // bytes of the block, so nothing past the payload is touched).
    uint32_t w[2][9];
    bool odd[2], live[2];
    __device__ void load(const uint8_t* W, int64_t rb, int n0, int N, int k0, int K) {
        const int t = threadIdx.x;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int u = t + 256 * it, row = u >> 2, kb = (k0 >> 5) + (u & 3);
            live[it] = kb < (K >> 5);
            const int n = min(n0 + row, N - 1);
            const uintptr_t a = reinterpret_cast<uintptr_t>(W + int64_t(n) * rb + 34 * int64_t(live[it] ? kb : 0));
            odd[it] = (a & 2) != 0;
            const uint32_t* p = reinterpret_cast<const uint32_t*>(a & ~uintptr_t(3));
#pragma unroll
            for (int i = 0; i < 9; ++i) w[it][i] = p[i];
        }
    }
    __device__ void store(int8_t* Bs, float (*dws)[BN], float (*)[BN], int) const {
        const int t = threadIdx.x;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int u = t + 256 * it, row = u >> 2, bi = u & 3;
            // block at 4-byte offset 2 (odd): d in the high half of dword 0, codes in dwords 1..8;
            // at offset 0: d in the low half, codes start at byte 2
            uint32_t c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = odd[it] ? w[it][i + 1] : align_byte(w[it][i + 1], w[it][i], 2);
            const float d = half_bits_to_float(odd[it] ? (w[it][0] >> 16) : (w[it][0] & 0xFFFFu));
            const uint32_t keep = live[it] ? 0xFFFFFFFFu : 0u;   // blocks past K contribute nothing
            *reinterpret_cast<uint4*>(Bs + row * LDA + 32 * bi) =
                make_uint4(c[0] & keep, c[1] & keep, c[2] & keep, c[3] & keep);
            *reinterpret_cast<uint4*>(Bs + row * LDA + 32 * bi + 16) =
                make_uint4(c[4] & keep, c[5] & keep, c[6] & keep, c[7] & keep);
            dws[bi][row] = live[it] ? d : 0.f;
        }
    }
};

template <> struct WeightRegs<kQ6_K> {
    // Thread t owns pieces u = t + 256 i (i < 4): row u/8, part p = u%8, which holds the
    // values 128h + 32tt + l, l in [4p, 4p+4), tt < 4, of super-block half h.  Thread
    // t < 128 also owns row t's 8 sub-scales of this half and d.
    uint32_t ql0[4], ql1[4], qh[4];
    uint32_t s0, s1, dbits;
    __device__ void load(const uint8_t* W, int64_t rb, int n0, int N, int k0, int) {
        const int t = threadIdx.x, sb = k0 >> 8, h = (k0 >> 7) & 1;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int u = t + 256 * it, row = u >> 3, p = u & 7;
            const int n = min(n0 + row, N - 1);
            const uint8_t* blk = W + int64_t(n) * rb + 210 * sb;
            ql0[it] = load_u32_a2(blk + 64 * h + 4 * p);
            ql1[it] = load_u32_a2(blk + 64 * h + 32 + 4 * p);
            qh[it] = load_u32_a2(blk + 128 + 32 * h + 4 * p);
        }
        const int n = min(n0 + (t & (BN - 1)), N - 1);
        const uint8_t* blk = W + int64_t(n) * rb + 210 * sb;
        s0 = load_u32_a2(blk + 192 + 8 * h);
        s1 = load_u32_a2(blk + 192 + 8 * h + 4);
        dbits = load_u16(blk + 208);
    }
    __device__ void store(int8_t* Bs, float (*dws)[BN], float (*)[BN], int) const {
        const int t = threadIdx.x;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int u = t + 256 * it, row = u >> 3, p = u & 7;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const uint32_t src = (tt & 1) ? ql1[it] : ql0[it];
                const uint32_t low = (tt < 2 ? src : (src >> 4)) & 0x0F0F0F0Fu;
                const uint32_t high = (qh[it] >> (2 * tt)) & 0x03030303u;
                uint32_t code = low | (high << 4);
                // per byte: code - 32 as int8 ((c + 128) - 32, then flip the sign bit back)
                code = ((code | 0x80808080u) - 0x20202020u) ^ 0x80808080u;
                *reinterpret_cast<uint32_t*>(Bs + row * LDA + 32 * tt + 4 * p) = code;
            }
        }
        if (t < BN) {
            const float d = half_bits_to_float(dbits);
#pragma unroll
            for (int gi = 0; gi < 8; ++gi) {
                const uint32_t word = gi < 4 ? s0 : s1;
                dws[gi][t] = d * float(int32_t(word << (24 - 8 * (gi & 3))) >> 24);
            }
        }
    }
};

template <int QT>
struct StepRegs {
    uint4 a[4];        // activation codes of row t/2, bytes 64*(t%2) + 16i of the step
    float dx[NB];      // thread t < 128: block scales of row t
    int32_t sx[NB];    // Q4_K: block code sums of row t
    WeightRegs<QT> w;

    // Every load is unconditional, from an in-bounds address: values past K are
    // replaced by zeros when the registers are written to LDS.  (A load under a
    // branch would make the compiler wait for it right away.)
    __device__ void load(const uint8_t* W, int64_t rb, const int8_t* codes, const float* xscale,
                         const int32_t* xsum, int m0, int n0, int M, int N, int K, int k0) {
        const int t = threadIdx.x;
        const int KB = K >> 5;
        const int ma = min(m0 + (t >> 1), M - 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kk = min(k0 + 64 * (t & 1) + 16 * i, K - 16);
            a[i] = *reinterpret_cast<const uint4*>(codes + int64_t(ma) * K + kk);
        }
        const int ms = min(m0 + (t & (BM - 1)), M - 1);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int kb = min((k0 >> 5) + b, KB - 1);
            dx[b] = xscale[int64_t(ms) * KB + kb];
            if constexpr (QT == kQ4_K) sx[b] = xsum[int64_t(ms) * KB + kb];
        }
        w.load(W, rb, n0, N, k0, K);
    }

    __device__ void store(int8_t* As, int8_t* Bs, float (*dxs)[BM], float (*txs)[BM], float (*dws)[BN],
                          float (*mws)[BN], int k0, int K) const {
        const int t = threadIdx.x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int kk = 64 * (t & 1) + 16 * i;
            *reinterpret_cast<uint4*>(As + (t >> 1) * LDA + kk) = (k0 + kk < K) ? a[i] : make_uint4(0, 0, 0, 0);
        }
        if (t < BM) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const bool in = k0 + 32 * b < K;
                dxs[b][t] = in ? dx[b] : 0.f;
                if constexpr (QT == kQ4_K) txs[b][t] = in ? dx[b] * float(sx[b]) : 0.f;
            }
        }
        w.store(Bs, dws, mws, k0);
    }
};

// ------------------------------------------------------------------ kernel
template <int QT, bool DUMP>
__global__ __launch_bounds__(256, 2) void mmq_kernel(const uint8_t* __restrict__ W,
                                                     const int8_t* __restrict__ codes,
                                                     const float* __restrict__ xscale,
                                                     const int32_t* __restrict__ xsum,
                                                     float* __restrict__ Y, int32_t* __restrict__ dots,
                                                     int M, int N, int K, int64_t row_bytes,
                                                     int tiles_m, int tiles_n, int splits, int total_steps) {
    constexpr int NG = Groups<QT>::per_step;
    __shared__ __attribute__((aligned(16))) int8_t As[BM * LDA];
    __shared__ __attribute__((aligned(16))) int8_t Bs[BN * LDA];
    __shared__ __attribute__((aligned(16))) float dxs[NB][BM];
    __shared__ __attribute__((aligned(16))) float txs[NB][BM];
    __shared__ __attribute__((aligned(16))) float dws[NG][BN];
    __shared__ __attribute__((aligned(16))) float mws[NB][BN];

    // XCD-aware order: workgroups that land on one XCD take consecutive logical ids, and
    // consecutive ids are the M-tiles of one (split, N-tile), which read the same weights.
    const int bid = blockIdx.x;
    const int total = int(gridDim.x);
    int logical = bid;
    if (total % kXcds == 0) logical = (bid % kXcds) * (total / kXcds) + bid / kXcds;
    const int tm = logical % tiles_m;
    const int tn = (logical / tiles_m) % tiles_n;
    const int split = logical / (tiles_m * tiles_n);
    const int m0 = tm * BM, n0 = tn * BN;
    // K range of this split: steps [s0, s1) of KS values; split-K partials go to slice
    // `split` of the partial buffer (Y itself when there is one split).
    const int kbeg = int(int64_t(split) * total_steps / splits) * KS;
    const int kend = min(int(int64_t(split + 1) * total_steps / splits) * KS, K);
    if (splits > 1 && !DUMP) Y += int64_t(split) * M * N;

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int g = lane >> 5;   // lane group: which half of a block's K this lane feeds
    const int r32 = lane & 31;
    const int KB = K >> 5;

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    StepRegs<QT> regs;
    regs.load(W, row_bytes, codes, xscale, xsum, m0, n0, M, N, K, kbeg);

    for (int k0 = kbeg; k0 < kend; k0 += KS) {
        __syncthreads();   // the previous step's LDS reads are done
        regs.store(As, Bs, dxs, txs, dws, mws, k0, K);
        __syncthreads();
        if (k0 + KS < kend) regs.load(W, row_bytes, codes, xscale, xsum, m0, n0, M, N, K, k0 + KS);

        if constexpr (QT != kQ6_K) {
#pragma unroll
            for (int p = 0; p < NB / 2; ++p) {   // block pair (2p, 2p+1)
                float dxo[2], dwo[2];
                v4i af[2][2], bf[2][2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    dxo[i] = dxs[2 * p + g][64 * wm + 32 * i + r32];
                    dwo[i] = dws[2 * p + g][64 * wn + 32 * i + r32];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int b = 2 * p + e;
                        af[i][e] = *reinterpret_cast<const v4i*>(As + (64 * wm + 32 * i + r32) * LDA + 32 * b + 16 * g);
                        bf[i][e] = *reinterpret_cast<const v4i*>(Bs + (64 * wn + 32 * i + r32) * LDA + 32 * b + 16 * g);
                    }
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const v32f z32 = {};
                        const v16i zi = {};
                        // element scales of block 2p (S[0..15]) and 2p+1 (S[16..31])
                        const v32f S = __builtin_amdgcn_mfma_f32_32x32x1f32(dxo[i], dwo[j], z32, 0, 0, 0);
                        const v16i D0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i][0], bf[j][0], zi, 0, 0, 0);
                        const v16i D1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i][1], bf[j][1], zi, 0, 0, 0);
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            acc[i][j][v] = fmaf(float(D0[v]), S[v], acc[i][j][v]);
                            acc[i][j][v] = fmaf(float(D1[v]), S[16 + v], acc[i][j][v]);
                        }
                        if constexpr (DUMP) {
                            const int nn = n0 + 64 * wn + 32 * j + r32;
                            const int kb = (k0 >> 5) + 2 * p;
#pragma unroll
                            for (int v = 0; v < 16; ++v) {
                                const int m = m0 + 64 * wm + 32 * i + acc_row(v, g);
                                if (m < M && nn < N) {
                                    const int64_t o = (int64_t(m) * N + nn) * KB + kb;
                                    if (kb < KB) dots[o] = D0[v];
                                    if (kb + 1 < KB) dots[o + 1] = D1[v];
                                }
                            }
                        }
                    }
            }
            if constexpr (QT == kQ4_K) {
                // min term: acc += sum_b txs[b][m] * mws[b][n] over the step's 4 blocks, 2 per MFMA
#pragma unroll
                for (int p = 0; p < NB / 2; ++p) {
                    float to[2], mo[2];
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        to[i] = txs[2 * p + g][64 * wm + 32 * i + r32];
                        mo[i] = mws[2 * p + g][64 * wn + 32 * i + r32];
                    }
#pragma unroll
                    for (int i = 0; i < 2; ++i)
#pragma unroll
                        for (int j = 0; j < 2; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(to[i], mo[j], acc[i][j], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                // block b as two 16-value groups 2b, 2b+1 with their own sub-scales
                long alo[2], ahi[2], blo[2], bhi[2];
                float dxe[2], dwo[2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int8_t* ap = As + (64 * wm + 32 * i + r32) * LDA + 32 * b + 8 * g;
                    alo[i] = *reinterpret_cast<const long*>(ap);
                    ahi[i] = *reinterpret_cast<const long*>(ap + 16);
                    const int8_t* bp = Bs + (64 * wn + 32 * i + r32) * LDA + 32 * b + 8 * g;
                    blo[i] = *reinterpret_cast<const long*>(bp);
                    bhi[i] = *reinterpret_cast<const long*>(bp + 16);
                    dxe[i] = dxs[b][64 * wm + 32 * i + r32];
                    dwo[i] = dws[2 * b + g][64 * wn + 32 * i + r32];
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const v32f z32 = {};
                        const v16i zi = {};
                        // element scales of group 2b (S[0..15]) and 2b+1 (S[16..31]): one dx, own d*s
                        const v32f S = __builtin_amdgcn_mfma_f32_32x32x1f32(dxe[i], dwo[j], z32, 0, 0, 0);
                        const v16i Dl = __builtin_amdgcn_mfma_i32_32x32x16_i8(alo[i], blo[j], zi, 0, 0, 0);
                        const v16i Dh = __builtin_amdgcn_mfma_i32_32x32x16_i8(ahi[i], bhi[j], zi, 0, 0, 0);
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            acc[i][j][v] = fmaf(float(Dl[v]), S[v], acc[i][j][v]);
                            acc[i][j][v] = fmaf(float(Dh[v]), S[16 + v], acc[i][j][v]);
                        }
                        if constexpr (DUMP) {
                            const int nn = n0 + 64 * wn + 32 * j + r32;
                            const int kb = (k0 >> 5) + b;
#pragma unroll
                            for (int v = 0; v < 16; ++v) {
                                const int m = m0 + 64 * wm + 32 * i + acc_row(v, g);
                                if (m < M && nn < N && kb < KB) {
                                    const int64_t o = (int64_t(m) * N + nn) * (2 * KB) + 2 * kb;
                                    dots[o] = Dl[v];
                                    dots[o + 1] = Dh[v];
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

// Sum of the split-K partials P[splits][count] in split order (deterministic).
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ P, float* __restrict__ Y,
                                                            int64_t count, int splits) {
    const int64_t stride = int64_t(gridDim.x) * 256;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < count; i += stride) {
        float acc = P[i];
        for (int s = 1; s < splits; ++s) acc += P[int64_t(s) * count + i];
        Y[i] = acc;
    }
}

template <int QT>
hipError_t launch_typed(const uint8_t* W, const int8_t* codes, const float* xs, const int32_t* xsum,
                        float* Y, int32_t* dots, float* partial, int64_t M, int64_t N, int64_t K,
                        int64_t row_bytes, hipStream_t s) {
    const MmqPlan plan = mmq_plan(QT, M, N, K);
    const int tiles_m = int((M + BM - 1) / BM);
    const int tiles_n = int((N + BN - 1) / BN);
    const int total = tiles_m * tiles_n * plan.splits;
    if (dots) {
        hipLaunchKernelGGL((mmq_kernel<QT, true>), dim3(total), dim3(256), 0, s, W, codes, xs, xsum, Y, dots,
                           int(M), int(N), int(K), row_bytes, tiles_m, tiles_n, plan.splits, plan.steps);
        return hipGetLastError();
    }
    float* out = plan.splits > 1 ? partial : Y;
    hipLaunchKernelGGL((mmq_kernel<QT, false>), dim3(total), dim3(256), 0, s, W, codes, xs, xsum, out, dots,
                       int(M), int(N), int(K), row_bytes, tiles_m, tiles_n, plan.splits, plan.steps);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || plan.splits == 1) return e;
    const int64_t count = M * N;
    const int64_t blocks = std::min<int64_t>((count + 255) / 256, 4096);
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, partial, Y, count,
                       plan.splits);
    return hipGetLastError();
}

}  // namespace

MmqPlan mmq_plan(int /*type*/, int64_t M, int64_t N, int64_t K) {
    // Enough workgroups to fill the chip: when the output has fewer tiles than about
    // 3/4 of kTargetWorkgroups, K is split so that tiles x splits comes near it, with at
    // least kMinStepsPerSplit K-steps per split.  A function of the shape alone, so the
    // result does not depend on the device.
    MmqPlan p;
    p.steps = int((K + KS - 1) / KS);
    p.splits = 1;
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    if (tiles * 4 < int64_t(kTargetWorkgroups) * 3) {
        const int64_t want = kTargetWorkgroups / tiles;
        p.splits = int(std::max<int64_t>(1, std::min<int64_t>(want, p.steps / kMinStepsPerSplit)));
    }
    return p;
}

size_t mmq_scratch_bytes(int type, int64_t M, int64_t N, int64_t K) {
    const MmqPlan p = mmq_plan(type, M, N, K);
    return p.splits > 1 ? size_t(p.splits) * size_t(M) * size_t(N) * sizeof(float) : 0;
}

hipError_t launch_mmq(int type, const uint8_t* W, const int8_t* codes, const float* xs, const int32_t* xsum,
                      float* Y, int32_t* dots, float* partial, int64_t M, int64_t N, int64_t K, hipStream_t s,
                      const char** name) {
    switch (type) {
        case kQ8_0:
            *name = "mmq<q8_0>";
            return launch_typed<kQ8_0>(W, codes, xs, xsum, Y, dots, partial, M, N, K, (K / 32) * 34, s);
        case kQ4_K:
            *name = "mmq<q4_K>";
            return launch_typed<kQ4_K>(W, codes, xs, xsum, Y, dots, partial, M, N, K, (K / 256) * 144, s);
        case kQ6_K:
            *name = "mmq<q6_K>";
            return launch_typed<kQ6_K>(W, codes, xs, xsum, Y, dots, partial, M, N, K, (K / 256) * 210, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mq
