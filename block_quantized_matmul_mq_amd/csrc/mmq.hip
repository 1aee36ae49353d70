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
// and walks its K range in steps of 128 values (4 blocks); each wave owns 2 x 2
// MFMA tiles of 32 x 32.  All tile data sits in LDS, double-buffered, so one
// barrier per step separates the buffer being read from the one being filled:
//   * activation codes and block scales/sums go global -> LDS directly
//     (buffer_load ... lds), with no registers in between;
//   * weight bytes are loaded into registers one step ahead and unpacked into
//     LDS as int8 codes (Q4_K 0..15, Q6_K code-32, Q8_0 q) plus f32 per-block
//     factors.
// LDS tiles are chunk-major (16-byte chunk c of every row, then chunk c+1), so a
// fragment read of 32 consecutive rows is 512 contiguous bytes.
//
// Per block pair and 32 x 32 tile the matrix unit does all the multiplies it
// can, so the vector ALU does two operations per output element and block
// (convert, fused multiply-add):
//   * v_mfma_i32_32x32x32_i8 forms the exact block dots D
//     (v_mfma_i32_32x32x16_i8 per 16-value group for Q6_K);
//   * v_mfma_f32_32x32x1_2b_f32 forms the two outer products dx (x) dw of a pair
//     of blocks: the f32 scale of every element of both blocks;
//   * the vector ALU accumulates acc += float(D) * scale;
//   * for Q4_K the min term sum_b (dx S)[m][b] * mw[n][b] is a small GEMM over
//     the step's 4 blocks, accumulated straight into acc by one
//     v_mfma_f32_32x32x16_bf16 per tile: both factors are split into two bf16
//     terms (hi + lo, together 16 significant bits) and the three products
//     hi*hi + hi*lo + lo*hi are summed in f32, so the term keeps a relative
//     error below 2^-16.  (An f32 MFMA here would not overlap the vector ALU of
//     the other wave on the SIMD; bf16 and int8 MFMAs do.)
// The tile products of a step are software-pipelined: the matrix-unit work of
// product k+1 is issued before the vector work of product k, so the two units
// run side by side within a wave.
//
// Workgroups are numbered so that the ones sharing a weight tile run on the
// same XCD (consecutive workgroup ids are dealt round-robin to the 8 XCDs, each
// with its own L2): a weight tile then comes from HBM once per XCD.
#include <algorithm>
#include <type_traits>

#include "mmq_splitk.h"
#include "mq_device.h"
#include "mq_internal.h"
#include "weight_units.h"

namespace mq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int BN = 128;         // output tile columns (weight rows)
constexpr int KS = 128;        // K values per step (bytes per LDS row)
constexpr int NB = KS / 32;    // 32-blocks per step
constexpr int kXcds = 8;
constexpr int kTargetWorkgroups = 512;   // two resident 256-thread workgroups on each of 256 CUs
constexpr int kMinStepsPerSplit = 2;
constexpr int kSmallM = 32;              // M up to this uses 32-row output tiles
constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource: 32-bit data format, no swizzle

template <int QT> struct Groups { static constexpr int per_step = NB; };
template <> struct Groups<kQ6_K> { static constexpr int per_step = 2 * NB; };

// Output tile rows: 128 for prefill-sized products, 32 for small M (at most 32 activation
// rows, where a 128-row tile would be mostly padding) and for products whose 128-row tiles
// would not fill half the chip (a small N: four times as many tiles, so fewer K cuts).
// Waves: WM x WN, each owning TI x TJ MFMA tiles of 32 x 32.
template <int BM_>
struct TileShape {
    static constexpr int BM = BM_;
    static constexpr int WM = BM_ == 128 ? 2 : 1;
    static constexpr int WN = 4 / WM;
    static constexpr int TI = BM_ / (32 * WM);
    static constexpr int TJ = BN / (32 * WN);
};

// LDS tiles are chunk-major: 16-byte chunk c (values 16c..16c+15 of the step) of row r
// sits at c * 16 * rows + r * 16.  A fragment read (32 consecutive rows, one chunk) is
// then 512 contiguous bytes, free of bank conflicts, and every address is a per-lane
// base plus a compile-time offset.
template <int ROWS>
__device__ __forceinline__ int chk(int r, int c) { return c * (ROWS * 16) + r * 16; }

// Row index (within a 32-row MFMA tile) of accumulator element v for lane group g = lane / 32.
__device__ __forceinline__ int acc_row(int v, int g) { return 8 * (v >> 2) + 4 * g + (v & 3); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kBufferWord3);
}

// x as two bf16 terms, hi = bf16(x) and lo = bf16(x - hi) (round to nearest even), packed as
// hi | lo << 16; hi + lo carries 16 significant bits of x.
__device__ __forceinline__ uint32_t bf16_hilo(float x) {
    const __bf16 hi = static_cast<__bf16>(x);
    const __bf16 lo = static_cast<__bf16>(x - static_cast<float>(hi));
    return uint32_t(__builtin_bit_cast(uint16_t, hi)) | (uint32_t(__builtin_bit_cast(uint16_t, lo)) << 16);
}

// Wait for every outstanding vector-memory operation of this wave (LDS-direct loads included).
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int QT, int BM>
struct Smem {
    int8_t A[2][BM * KS];                               // activation codes
    int8_t B[2][BN * KS];                               // weight codes
    float dx[2][NB][BM];                                // activation block scales
    uint32_t tx[2][has_min_term<QT>() ? NB : 1][BM];    // min types: bf16_hilo(dx * code sum) per block
    float dw[2][Groups<QT>::per_step][BN];              // weight scale per block (per group, Q6_K)
    uint32_t mw[2][has_min_term<QT>() ? NB : 1][BN];    // bf16_hilo(-dmin * m) (K-quants) or m per block
};

// ------------------------------------------------------------------ weight staging
// Raw weight bytes of one K-step, held in registers from the load (issued a step
// ahead) to the LDS write.  Rows past N re-read row N-1: their outputs are never stored.
template <int QT> struct WeightRegs;

template <> struct WeightRegs<kQ4_K> {
    // Thread t owns row t % 128 and, of the 4 16-byte code chunks that hold this step's
    // 128 values (half = which half of the super-block the step covers), chunks p0 and
    // p0 + 2 with p0 = t / 128; and the row's 16-byte header (d, dmin, packed scales).
    // Chunk p holds the low nibbles (values 16p' ..) of sub-block 2c and the high nibbles
    // of sub-block 2c + 1, c = 2 half + p / 2.  A wave writes one chunk of 64 consecutive
    // rows at a time: 1 KB of contiguous LDS, no bank conflicts.
    uint4 q[2], hd;
    __device__ void load(const uint8_t* W, int64_t rb, int n0, int N, int k0, int, int bs, int bo) {
        const int t = threadIdx.x, sb = k0 >> 8, half = (k0 >> 7) & 1;
        const int n = min(n0 + (t & (BN - 1)), N - 1);
        const uint8_t* blk = W + int64_t(n) * rb + 144 * sb;
        const int p0 = t >> 7;
#pragma unroll
        for (int it = 0; it < 2; ++it)
            q[it] = *reinterpret_cast<const uint4*>(blk + 16 + 16 * (4 * half + p0 + 2 * it));
        hd = *reinterpret_cast<const uint4*>(blk);
    }
    template <int BM>
    __device__ void store(Smem<kQ4_K, BM>& sm, int buf, int k0) const {
        const int t = threadIdx.x, half = (k0 >> 7) & 1;
        const int row = t & (BN - 1), p0 = t >> 7;
        int8_t* Bs = sm.B[buf];
        const float d = half_bits_to_float(hd.x & 0xFFFFu);
        const float dmin = half_bits_to_float(hd.x >> 16);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int p = p0 + 2 * it;          // chunk within the step's 64 code bytes
            const int c = p >> 1, h = p & 1;    // 64-value group c of the step, piece h of it
            const uint4 v = q[it];
            const uint4 lo = make_uint4(v.x & 0x0F0F0F0Fu, v.y & 0x0F0F0F0Fu, v.z & 0x0F0F0F0Fu, v.w & 0x0F0F0F0Fu);
            const uint4 hi = make_uint4((v.x >> 4) & 0x0F0F0F0Fu, (v.y >> 4) & 0x0F0F0F0Fu,
                                        (v.z >> 4) & 0x0F0F0F0Fu, (v.w >> 4) & 0x0F0F0F0Fu);
            // group c holds values 64c..64c+63 of the step: low nibbles the first 32, high nibbles
            // the next 32; piece h is 16 bytes, i.e. 16-value chunks 4c + h (low) and 4c + h + 2 (high)
            *reinterpret_cast<uint4*>(Bs + chk<BN>(row, 4 * c + h)) = lo;
            *reinterpret_cast<uint4*>(Bs + chk<BN>(row, 4 * c + h + 2)) = hi;
            // this thread also decodes step block jb = 2c + h (sub-block 4 half + jb of the
            // super-block); the branch inside is uniform (it depends on half only)
            const int jb = 2 * c + h;
            uint32_t sc, mn;
            q4k_scale_min(hd.y, hd.z, hd.w, 4 * half + jb, sc, mn);
            sm.dw[buf][jb][row] = d * float(sc);
            sm.mw[buf][jb][row] = bf16_hilo(-(dmin * float(mn)));
        }
    }
};

template <> struct WeightRegs<kQ8_0> {
    // Thread t owns row t % 128 and blocks b0 and b0 + 2 of this step, b0 = t / 128, each
    // read as the 9 naturally aligned dwords that cover its 34 bytes (every one of them
    // holds bytes of the block, so nothing past the payload is touched).  A wave writes
    // one chunk of 64 consecutive rows at a time.
    uint32_t w[2][9];
    bool odd[2], live[2];
    __device__ void load(const uint8_t* W, int64_t rb, int n0, int N, int k0, int K, int bs, int bo) {
        const int t = threadIdx.x;
        const int n = min(n0 + (t & (BN - 1)), N - 1);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int kb = (k0 >> 5) + (t >> 7) + 2 * it;
            live[it] = kb < (K >> 5);
            const uintptr_t a =
                reinterpret_cast<uintptr_t>(W + int64_t(n) * rb + int64_t(bs) * (live[it] ? kb : 0) + bo);
            odd[it] = (a & 2) != 0;
            const uint32_t* p = reinterpret_cast<const uint32_t*>(a & ~uintptr_t(3));
#pragma unroll
            for (int i = 0; i < 9; ++i) w[it][i] = p[i];
        }
    }
    template <int BM>
    __device__ void store(Smem<kQ8_0, BM>& sm, int buf, int) const {
        const int t = threadIdx.x;
        const int row = t & (BN - 1);
        int8_t* Bs = sm.B[buf];
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int bi = (t >> 7) + 2 * it;
            // block at 4-byte offset 2 (odd): d in the high half of dword 0, codes in dwords 1..8;
            // at offset 0: d in the low half, codes start at byte 2
            uint32_t c[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) c[i] = odd[it] ? w[it][i + 1] : align_byte(w[it][i + 1], w[it][i], 2);
            const float d = half_bits_to_float(odd[it] ? (w[it][0] >> 16) : (w[it][0] & 0xFFFFu));
            const uint32_t keep = live[it] ? 0xFFFFFFFFu : 0u;   // blocks past K contribute nothing
            *reinterpret_cast<uint4*>(Bs + chk<BN>(row, 2 * bi)) =
                make_uint4(c[0] & keep, c[1] & keep, c[2] & keep, c[3] & keep);
            *reinterpret_cast<uint4*>(Bs + chk<BN>(row, 2 * bi + 1)) =
                make_uint4(c[4] & keep, c[5] & keep, c[6] & keep, c[7] & keep);
            sm.dw[buf][bi][row] = live[it] ? d : 0.f;
        }
    }
};

template <> struct WeightRegs<kQ5_K> {
    // As Q4_K (chunks p0 and p0 + 2 of the step's 64 code bytes, and the row's header),
    // plus the 16 high-bit bytes qh[16 (p0 % 2) ..]: chunk p covers byte l of its 64-value
    // group c, whose two sub-blocks take bits 2c and 2c + 1 of qh[l].
    uint4 q[2], hd, qh;
    __device__ void load(const uint8_t* W, int64_t rb, int n0, int N, int k0, int, int, int) {
        const int t = threadIdx.x, sb = k0 >> 8, half = (k0 >> 7) & 1;
        const int n = min(n0 + (t & (BN - 1)), N - 1);
        const uint8_t* blk = W + int64_t(n) * rb + 176 * sb;
        const int p0 = t >> 7;
#pragma unroll
        for (int it = 0; it < 2; ++it)
            q[it] = *reinterpret_cast<const uint4*>(blk + 48 + 16 * (4 * half + p0 + 2 * it));
        hd = *reinterpret_cast<const uint4*>(blk);
        qh = *reinterpret_cast<const uint4*>(blk + 16 + 16 * (p0 & 1));
    }
    template <int BM>
    __device__ void store(Smem<kQ5_K, BM>& sm, int buf, int k0) const {
        const int t = threadIdx.x, half = (k0 >> 7) & 1;
        const int row = t & (BN - 1), p0 = t >> 7;
        int8_t* Bs = sm.B[buf];
        const float d = half_bits_to_float(hd.x & 0xFFFFu);
        const float dmin = half_bits_to_float(hd.x >> 16);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int p = p0 + 2 * it;
            const int c = p >> 1, h = p & 1;
            const uint32_t s = 2u * uint32_t(2 * half + c);   // qh bit of the group's first sub-block
            const uint4 v = q[it];
            auto hb = [&](uint32_t w, uint32_t b) { return ((w >> b) & 0x01010101u) << 4; };
            const uint4 lo = make_uint4((v.x & 0x0F0F0F0Fu) | hb(qh.x, s), (v.y & 0x0F0F0F0Fu) | hb(qh.y, s),
                                        (v.z & 0x0F0F0F0Fu) | hb(qh.z, s), (v.w & 0x0F0F0F0Fu) | hb(qh.w, s));
            const uint4 hi = make_uint4(((v.x >> 4) & 0x0F0F0F0Fu) | hb(qh.x, s + 1),
                                        ((v.y >> 4) & 0x0F0F0F0Fu) | hb(qh.y, s + 1),
                                        ((v.z >> 4) & 0x0F0F0F0Fu) | hb(qh.z, s + 1),
                                        ((v.w >> 4) & 0x0F0F0F0Fu) | hb(qh.w, s + 1));
            *reinterpret_cast<uint4*>(Bs + chk<BN>(row, 4 * c + h)) = lo;
            *reinterpret_cast<uint4*>(Bs + chk<BN>(row, 4 * c + h + 2)) = hi;
            const int jb = 2 * c + h;
            uint32_t sc, mn;
            q4k_scale_min(hd.y, hd.z, hd.w, 4 * half + jb, sc, mn);
            sm.dw[buf][jb][row] = d * float(sc);
            sm.mw[buf][jb][row] = bf16_hilo(-(dmin * float(mn)));
        }
    }
};

// Q4_0 / Q4_1 / Q5_0 / Q5_1: thread t owns row t % 128 and blocks b0 and b0 + 2 of this
// step, b0 = t / 128 (as Q8_0), read through the 32-value unit loader.  The codes go to LDS
// as int8: code - offset for Q4_0 / Q5_0 (signed), the code itself for Q4_1 / Q5_1 (whose
// min m rides on the activation block's code sum).  Blocks past K contribute nothing.
template <int QT>
struct LegacyRegs {
    RawLegacy<QT> blk[2];
    bool live[2];
    __device__ void load(const uint8_t* W, int64_t rb, int n0, int N, int k0, int K, int, int) {
        const int t = threadIdx.x;
        const int n = min(n0 + (t & (BN - 1)), N - 1);
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int kb = (k0 >> 5) + (t >> 7) + 2 * it;
            live[it] = kb < (K >> 5);
            blk[it].load(W + int64_t(n) * rb, live[it] ? kb : 0, 0, 0);
        }
    }
    template <int BM>
    __device__ void store(Smem<QT, BM>& sm, int buf, int) const {
        const int t = threadIdx.x;
        const int row = t & (BN - 1);
        int8_t* Bs = sm.B[buf];
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int bi = (t >> 7) + 2 * it;
            uint32_t c[8];
            blk[it].codes(c);
            const uint32_t keep = live[it] ? 0xFFFFFFFFu : 0u;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if constexpr (Legacy<QT>::kOffset != 0)   // per byte: (c + 128 - offset) with the sign bit flipped back
                    c[i] = ((c[i] | 0x80808080u) - 0x01010101u * uint32_t(Legacy<QT>::kOffset)) ^ 0x80808080u;
                c[i] &= keep;
            }
            *reinterpret_cast<uint4*>(Bs + chk<BN>(row, 2 * bi)) = make_uint4(c[0], c[1], c[2], c[3]);
            *reinterpret_cast<uint4*>(Bs + chk<BN>(row, 2 * bi + 1)) = make_uint4(c[4], c[5], c[6], c[7]);
            sm.dw[buf][bi][row] = live[it] ? blk[it].d() : 0.f;
            if constexpr (Legacy<QT>::kMin) sm.mw[buf][bi][row] = live[it] ? bf16_hilo(blk[it].m()) : 0u;
        }
    }
};
template <> struct WeightRegs<kQ4_0> : LegacyRegs<kQ4_0> {};
template <> struct WeightRegs<kQ4_1> : LegacyRegs<kQ4_1> {};
template <> struct WeightRegs<kQ5_0> : LegacyRegs<kQ5_0> {};
template <> struct WeightRegs<kQ5_1> : LegacyRegs<kQ5_1> {};

template <> struct WeightRegs<kQ6_K> {
    // Thread t owns pieces u = t + 256 i (i < 4): row u/8, part p = u%8, which holds the
    // values 128h + 32tt + l, l in [4p, 4p+4), tt < 4, of super-block half h.  Thread
    // t < 128 also owns row t's 8 sub-scales of this half and d.
    uint32_t ql0[4], ql1[4], qh[4];
    uint32_t s0, s1, dbits;
    __device__ void load(const uint8_t* W, int64_t rb, int n0, int N, int k0, int, int bs, int bo) {
        const int t = threadIdx.x, sb = k0 >> 8, h = (k0 >> 7) & 1;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int u = t + 256 * it, row = u >> 3, p = u & 7;
            const int n = min(n0 + row, N - 1);
            const uint8_t* blk = W + int64_t(n) * rb + bs * sb + bo;
            ql0[it] = load_u32_a2(blk + 64 * h + 4 * p);
            ql1[it] = load_u32_a2(blk + 64 * h + 32 + 4 * p);
            qh[it] = load_u32_a2(blk + 128 + 32 * h + 4 * p);
        }
        const int n = min(n0 + (t & (BN - 1)), N - 1);
        const uint8_t* blk = W + int64_t(n) * rb + bs * sb + bo;
        s0 = load_u32_a2(blk + 192 + 8 * h);
        s1 = load_u32_a2(blk + 192 + 8 * h + 4);
        dbits = load_u16(blk + 208);
    }
    template <int BM>
    __device__ void store(Smem<kQ6_K, BM>& sm, int buf, int) const {
        const int t = threadIdx.x;
        int8_t* Bs = sm.B[buf];
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
                // values 32tt + 4p .. +3 of the step: chunk 2tt + p/4, bytes 4(p%4)..
                *reinterpret_cast<uint32_t*>(Bs + chk<BN>(row, 2 * tt + (p >> 2)) + 4 * (p & 3)) = code;
            }
        }
        if (t < BN) {
            const float d = half_bits_to_float(dbits);
#pragma unroll
            for (int gi = 0; gi < 8; ++gi) {
                const uint32_t word = gi < 4 ? s0 : s1;
                sm.dw[buf][gi][t] = d * float(int32_t(word << (24 - 8 * (gi & 3))) >> 24);
            }
        }
    }
};

// ------------------------------------------------------------------ activation staging
// Activation codes and block scales of one K-step, loaded by each wave straight into
// LDS.  One buffer_load ... lds instruction writes 64 lanes x 16 (or 4) consecutive LDS
// bytes; each lane picks the global bytes that belong at its LDS slot.  Loads past the
// tile's last row return zeros (buffer range check).  The scales of the step form NB x BM
// dword slots, 64 per instruction: wave w issues instructions 2w and 2w+1 (those that
// exist); for Q4_K it also loads the matching code sums into registers, and after its
// loads have landed forms the min-term factor dx * sum of those slots itself (its own
// loads are complete after its own wait, before any barrier).
template <int QT, int BM>
struct ActDirect {
    static constexpr int kCodeIns = BM / 32;           // 1 KB code instructions per wave
    static constexpr int kScaleIns = NB * BM / 64;     // 64-dword scale instructions in all
    __amdgpu_buffer_rsrc_t rc, rs, ru;
    uint32_t voff_a[kCodeIns];   // codes: lane's byte offset per instruction
    uint32_t voff_s[2];          // scales / sums: lane's byte offset per instruction
    int32_t sums[2];             // Q4_K: code sums of the lane's two scale slots

    __device__ void init(const int8_t* codes, const float* xscale, const int32_t* xsum, int m0, int M, int K) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int rows = min(BM, M - m0);
        const int KB = K >> 5;
        rc = make_rsrc(codes + int64_t(m0) * K, int64_t(rows) * K);
        rs = make_rsrc(xscale + int64_t(m0) * KB, int64_t(rows) * KB * 4);
        ru = make_rsrc(xsum + int64_t(m0) * KB, int64_t(rows) * KB * 4);
#pragma unroll
        for (int i = 0; i < kCodeIns; ++i) {
            // instruction i of wave w fills LDS bytes 1024 (kCodeIns w + i) .. +1023 of the
            // chunk-major tile: chunk o / (16 BM), row (o % (16 BM)) / 16 for byte o
            const int o = 1024 * (kCodeIns * wave + i) + 16 * lane;
            const int c = o / (16 * BM), row = (o % (16 * BM)) / 16;
            voff_a[i] = uint32_t(row * K + 16 * c);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int slot = 64 * (2 * wave + j) + lane;   // block slot / BM, row slot % BM
            voff_s[j] = uint32_t(((slot % BM) * KB + slot / BM) * 4);
        }
    }

    __device__ void issue(Smem<QT, BM>& sm, int buf, int k0) {
        const int wave = threadIdx.x >> 6;
#pragma unroll
        for (int i = 0; i < kCodeIns; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rc, (lds_void*)(sm.A[buf] + 1024 * (kCodeIns * wave + i)), 16,
                                                     voff_a[i], uint32_t(k0), 0, 0);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (2 * wave + j < kScaleIns) {   // uniform
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(&sm.dx[buf][0][0] + 64 * (2 * wave + j)), 4,
                                                         voff_s[j], uint32_t(k0 >> 3), 0, 0);
                if constexpr (has_min_term<QT>())
                    sums[j] = __builtin_amdgcn_raw_buffer_load_b32(ru, voff_s[j], uint32_t(k0 >> 3), 0);
            }
        }
    }

    // after this wave's loads of the step in `buf` have landed
    __device__ void finish(Smem<QT, BM>& sm, int buf) const {
        if constexpr (has_min_term<QT>()) {
            const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (2 * wave + j < kScaleIns) {
                    const int slot = 64 * (2 * wave + j) + lane;
                    (&sm.tx[buf][0][0])[slot] = bf16_hilo((&sm.dx[buf][0][0])[slot] * float(sums[j]));
                }
            }
        }
    }
};

// ------------------------------------------------------------------ kernel
template <int QT, int BM, bool DUMP>
__global__ __launch_bounds__(256, 2) void mmq_kernel(const uint8_t* __restrict__ W,
                                                     const int8_t* __restrict__ codes,
                                                     const float* __restrict__ xscale,
                                                     const int32_t* __restrict__ xsum,
                                                     float* __restrict__ Y, int32_t* __restrict__ dots,
                                                     float* __restrict__ partial, unsigned* __restrict__ counters,
                                                     int M, int N, int K, int64_t row_bytes, int blk_stride,
                                                     int blk_off, int tiles_m, int full, int split_tiles, int splits,
                                                     int total_steps) {
    using T = TileShape<BM>;
    constexpr int TI = T::TI, TJ = T::TJ;
    __shared__ __attribute__((aligned(16))) Smem<QT, BM> sm;

    // Work split (MmqPlan): workgroups [0, full) own whole tiles 0..full-1; the remaining
    // split_tiles tiles are each cut into `splits` K ranges, one workgroup per range, whose
    // f32 partial tiles the range that finishes last sums (mmq_splitk.h).  Within each group
    // the ids are remapped so
    // that workgroups landing on one XCD take consecutive logical ids, and consecutive ids
    // are the M-tiles of one N-tile, which read the same weights.
    const int id = blockIdx.x;
    const bool whole = id < full;
    const int group = whole ? full : split_tiles * splits;
    const int j0 = whole ? id : id - full;
    const int jj = group % kXcds == 0 ? (j0 % kXcds) * (group / kXcds) + j0 / kXcds : j0;
    const int tile = whole ? jj : full + jj % split_tiles;
    const int split = whole ? 0 : jj / split_tiles;
    const int nsplit = whole ? 1 : splits;
    const int tm = tile % tiles_m;
    const int tn = tile / tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    // K range: steps [s0, s1) of KS values
    const int kbeg = int(int64_t(split) * total_steps / nsplit) * KS;
    const int kend = min(int(int64_t(split + 1) * total_steps / nsplit) * KS, K);

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = t >> 6;
    const int wm = wave / T::WN, wn = wave % T::WN;
    const int g = lane >> 5;   // lane group: which half of a block's K this lane feeds
    const int r32 = lane & 31;
    const int KB = K >> 5;

    v16f acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    ActDirect<QT, BM> act;
    act.init(codes, xscale, xsum, m0, M, K);
    WeightRegs<QT> wr;

    // prologue: step kbeg into buffer 0, step kbeg + KS in flight
    wr.load(W, row_bytes, n0, N, kbeg, K, blk_stride, blk_off);
    act.issue(sm, 0, kbeg);
    wait_vm_all();
    wr.store(sm, 0, kbeg);
    act.finish(sm, 0);
    __syncthreads();
    if (kbeg + KS < kend) {
        wr.load(W, row_bytes, n0, N, kbeg + KS, K, blk_stride, blk_off);
        act.issue(sm, 1, kbeg + KS);
    }

    // One K-step on LDS buffer BUF (a compile-time constant, so every LDS address is a
    // per-lane base plus an immediate offset); the loop alternates the two buffers.
    auto step = [&](auto buf_c, int k0) {
        constexpr int buf = decltype(buf_c)::value;
        const int8_t* As = sm.A[buf];
        const int8_t* Bs = sm.B[buf];
        const int arow0 = 32 * TI * wm + r32;   // + 32 i
        const int brow0 = 32 * TJ * wn + r32;   // + 32 j

        // Tile products of the step, k = (TI TJ) p + TJ i + j (block pair p, or block p for
        // Q6_K's two 16-value groups; tiles i, j).  Product k needs: S (the scale outer product, 32
        // regs) and two int32 dot tiles D0, D1 (16 regs each).  Pipeline: S of product k+1
        // is issued when product k starts; D0 of product k+1 as soon as product k has used
        // its D0, D1 likewise, so every matrix-unit result has a half product of vector work
        // to arrive in.
        constexpr int kTiles = TI * TJ;
        constexpr int kProducts = (QT == kQ6_K ? 4 : 2) * kTiles;
        v32f S[2];
        v16i D0, D1;
        // operands of the next product's dot tiles
        v4i na0, na1, nb0, nb1;   // 16-byte fragments (Q8_0, Q4_K)
        long la0, la1, lb0, lb1;  // 8-byte fragments (Q6_K)
        float sdx, sdw;           // the next product's scale-outer-product operands
        auto frag = [&](int k) {
            const int p = k / kTiles, i = (k / TJ) % TI, j = k % TJ;
            const int ar = arow0 + 32 * i, br = brow0 + 32 * j;
            if constexpr (QT != kQ6_K) {
                na0 = *reinterpret_cast<const v4i*>(As + chk<BM>(ar, 4 * p + g));
                na1 = *reinterpret_cast<const v4i*>(As + chk<BM>(ar, 4 * p + 2 + g));
                nb0 = *reinterpret_cast<const v4i*>(Bs + chk<BN>(br, 4 * p + g));
                nb1 = *reinterpret_cast<const v4i*>(Bs + chk<BN>(br, 4 * p + 2 + g));
                sdx = sm.dx[buf][2 * p + g][ar];   // block 2p + g (lane group g feeds block g of the pair)
            } else {
                la0 = *reinterpret_cast<const long*>(As + chk<BM>(ar, 2 * p) + 8 * g);
                la1 = *reinterpret_cast<const long*>(As + chk<BM>(ar, 2 * p + 1) + 8 * g);
                lb0 = *reinterpret_cast<const long*>(Bs + chk<BN>(br, 2 * p) + 8 * g);
                lb1 = *reinterpret_cast<const long*>(Bs + chk<BN>(br, 2 * p + 1) + 8 * g);
                sdx = sm.dx[buf][p][ar];           // one block scale for both groups
            }
            sdw = sm.dw[buf][2 * p + g][br];
        };
        // Q8_0 / Q4_K: element scales of block 2p (out[0..15]) and 2p+1 (out[16..31]);
        // Q6_K: of groups 2p (out[0..15]) and 2p+1 (out[16..31]) of block p
        auto scales = [&](v32f& out) {
            const v32f z32 = {};
            out = __builtin_amdgcn_mfma_f32_32x32x1f32(sdx, sdw, z32, 0, 0, 0);
        };
        auto dot0 = [&]() {
            const v16i zi = {};
            if constexpr (QT != kQ6_K) D0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(na0, nb0, zi, 0, 0, 0);
            else D0 = __builtin_amdgcn_mfma_i32_32x32x16_i8(la0, lb0, zi, 0, 0, 0);
        };
        auto dot1 = [&]() {
            const v16i zi = {};
            if constexpr (QT != kQ6_K) D1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(na1, nb1, zi, 0, 0, 0);
            else D1 = __builtin_amdgcn_mfma_i32_32x32x16_i8(la1, lb1, zi, 0, 0, 0);
        };
        // acc += float(D) * S-half h, and the block-dot export
        auto consume = [&](int k, const v32f& Sk, const v16i& D, int h) {
            const int p = k / kTiles, i = (k / TJ) % TI, j = k % TJ;
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = fmaf(float(D[v]), Sk[16 * h + v], acc[i][j][v]);
            // pin the accumulation here: without it the compiler sinks all vector work of
            // the step below the matrix-unit work, and the dot tiles pile up in registers
            asm volatile("" : "+v"(acc[i][j]));
            if constexpr (DUMP) {
                const int nn = n0 + brow0 + 32 * j;
                // Q8_0 / Q4_K: block 2p + h; Q6_K: group h of block p
                const int kb = (k0 >> 5) + (QT == kQ6_K ? p : 2 * p + h);
                const int G = QT == kQ6_K ? 2 * KB : KB;
                const int gi = QT == kQ6_K ? 2 * kb + h : kb;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = m0 + 32 * TI * wm + 32 * i + acc_row(v, g);
                    if (m < M && nn < N && kb < KB) dots[(int64_t(m) * N + nn) * G + gi] = D[v];
                }
            }
        };
        // Q4_K min term of tile (i, j) for the step's 4 blocks, acc += sum_b tx[m][b] * mw[n][b]:
        // one bf16 MFMA with K = 16 = 4 blocks x 4 slots; lane group g feeds blocks 2g, 2g+1,
        // slots (hi*hi, hi*lo, lo*hi, 0) from the hi | lo << 16 packs.
        auto min_term = [&](int i, int j) {
            if constexpr (has_min_term<QT>()) {
                const int ar = arow0 + 32 * i, br = brow0 + 32 * j;
                const uint32_t t0 = sm.tx[buf][2 * g][ar], t1 = sm.tx[buf][2 * g + 1][ar];
                const uint32_t w0 = sm.mw[buf][2 * g][br], w1 = sm.mw[buf][2 * g + 1][br];
                const v4i a = {int((t0 & 0xFFFFu) | (t0 << 16)), int(t0 >> 16), int((t1 & 0xFFFFu) | (t1 << 16)),
                               int(t1 >> 16)};
                const v4i b = {int(w0), int(w0 & 0xFFFFu), int(w1), int(w1 & 0xFFFFu)};
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                                    __builtin_bit_cast(v8bf, b), acc[i][j], 0, 0, 0);
            }
        };

        // Each product is cut into scheduling regions (sched_barrier) so that the matrix-unit
        // work of product k+1 sits between the two halves of product k's vector work.
        frag(0);
        scales(S[0]);
        dot0();
        dot1();
#pragma unroll
        for (int k = 0; k < kProducts; ++k) {
            const int cur = k & 1;
            const bool more = k + 1 < kProducts;
            if (more) frag(k + 1);
            __builtin_amdgcn_sched_barrier(0);
            consume(k, S[cur], D0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (more) {
                scales(S[cur ^ 1]);
                dot0();
            }
            __builtin_amdgcn_sched_barrier(0);
            consume(k, S[cur], D1, 1);
            __builtin_amdgcn_sched_barrier(0);
            if (more) dot1();
            __builtin_amdgcn_sched_barrier(0);
            if (has_min_term<QT>() && k / kTiles == 1) min_term((k / TJ) % TI, k % TJ);
        }
        // next step: its weight registers and LDS-direct loads were issued a step ago
        if (k0 + KS < kend) {
            wait_vm_all();
            wr.store(sm, buf ^ 1, k0 + KS);
            act.finish(sm, buf ^ 1);
        }
        __syncthreads();   // buffer `buf` is free, buffer `buf ^ 1` is complete
        if (k0 + 2 * KS < kend) {
            wr.load(W, row_bytes, n0, N, k0 + 2 * KS, K, blk_stride, blk_off);
            act.issue(sm, buf, k0 + 2 * KS);
        }
    };
    for (int k0 = kbeg;;) {
        step(std::integral_constant<int, 0>{}, k0);
        if ((k0 += KS) >= kend) break;
        step(std::integral_constant<int, 1>{}, k0);
        if ((k0 += KS) >= kend) break;
    }

    // Y store: for a fixed accumulator element the 32 lanes of a group write 32 consecutive n.
    // The block-dot export variant stores only the dots.
    if constexpr (DUMP) return;
    auto store = [&](int i, int j, const float* y) {
        const int n = n0 + 32 * TJ * wn + 32 * j + r32;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = m0 + 32 * TI * wm + 32 * i + acc_row(v, g);
            if (m < M && n < N) Y[int64_t(m) * N + n] = y[v];
        }
    };
    if (whole) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                float y[16];
#pragma unroll
                for (int v = 0; v < 16; ++v) y[v] = acc[i][j][v];
                store(i, j, y);
            }
        return;
    }
    // A split tile puts its partial into its range's slot, and the range that counts in last
    // sums all ranges' slots in range order into Y.
    constexpr uint32_t kSlotBytes = BM * BN * sizeof(float);
    const __amdgpu_buffer_rsrc_t slots =
        make_rsrc(partial + size_t(tile - full) * size_t(splits) * (BM * BN), int64_t(splits) * kSlotBytes);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; v += 4)
                splitk_put<256>(slots, uint32_t(split) * kSlotBytes, ((i * TJ + j) * 16 + v) / 4,
                                splitk_f4{acc[i][j][v], acc[i][j][v + 1], acc[i][j][v + 2], acc[i][j][v + 3]});
    // the ticket word: LDS that no thread touches after the last step's barrier
    if (!splitk_arrive(counters + (tile - full), splits, reinterpret_cast<unsigned*>(&sm.dx[0][0][0]))) return;
#pragma unroll
    for (int i = 0; i < TI; ++i) {   // one row of accumulator tiles at a time (registers)
        float y[TJ * 16];
        splitk_sum<TJ * 16, 256>(slots, kSlotBytes, splits, i * TJ * 4, y);
#pragma unroll
        for (int j = 0; j < TJ; ++j) store(i, j, y + 16 * j);
    }
}

// Explicit instantiations: the host-side launch stubs of these kernels are otherwise not
// emitted by this compiler when they are only named inside launch_shaped below.
#define MQ_MMQ_INSTANCE(QT, BM, DUMP)                                                                        \
    template __global__ void mmq_kernel<QT, BM, DUMP>(const uint8_t* __restrict__, const int8_t* __restrict__, \
                                                      const float* __restrict__, const int32_t* __restrict__,  \
                                                      float* __restrict__, int32_t* __restrict__,              \
                                                      float* __restrict__, unsigned* __restrict__, int, int, int, \
                                                      int64_t, int, int, int, int, int, int, int);
MQ_MMQ_INSTANCE(kQ5_K, 32, false)
MQ_MMQ_INSTANCE(kQ5_K, 128, false)
MQ_MMQ_INSTANCE(kQ5_K, 32, true)
MQ_MMQ_INSTANCE(kQ5_K, 128, true)
MQ_MMQ_INSTANCE(kQ4_0, 32, false)
MQ_MMQ_INSTANCE(kQ4_0, 128, false)
MQ_MMQ_INSTANCE(kQ4_0, 32, true)
MQ_MMQ_INSTANCE(kQ4_0, 128, true)
MQ_MMQ_INSTANCE(kQ4_1, 32, false)
MQ_MMQ_INSTANCE(kQ4_1, 128, false)
MQ_MMQ_INSTANCE(kQ4_1, 32, true)
MQ_MMQ_INSTANCE(kQ4_1, 128, true)
MQ_MMQ_INSTANCE(kQ5_0, 32, false)
MQ_MMQ_INSTANCE(kQ5_0, 128, false)
MQ_MMQ_INSTANCE(kQ5_0, 32, true)
MQ_MMQ_INSTANCE(kQ5_0, 128, true)
MQ_MMQ_INSTANCE(kQ5_1, 32, false)
MQ_MMQ_INSTANCE(kQ5_1, 128, false)
MQ_MMQ_INSTANCE(kQ5_1, 32, true)
MQ_MMQ_INSTANCE(kQ5_1, 128, true)
MQ_MMQ_INSTANCE(kQ8_0, 32, false)
MQ_MMQ_INSTANCE(kQ8_0, 128, false)
MQ_MMQ_INSTANCE(kQ4_K, 32, false)
MQ_MMQ_INSTANCE(kQ4_K, 128, false)
MQ_MMQ_INSTANCE(kQ6_K, 32, false)
MQ_MMQ_INSTANCE(kQ6_K, 128, false)
MQ_MMQ_INSTANCE(kQ8_0, 32, true)
MQ_MMQ_INSTANCE(kQ8_0, 128, true)
MQ_MMQ_INSTANCE(kQ4_K, 32, true)
MQ_MMQ_INSTANCE(kQ4_K, 128, true)
MQ_MMQ_INSTANCE(kQ6_K, 32, true)
MQ_MMQ_INSTANCE(kQ6_K, 128, true)
#undef MQ_MMQ_INSTANCE

template <int QT, int BM>
hipError_t launch_shaped(const uint8_t* W, const int8_t* codes, const float* xs, const int32_t* xsum, float* Y,
                         int32_t* dots, float* partial, unsigned* counters, int64_t M, int64_t N, int64_t K,
                         BlockLayout lay, const MmqPlan& plan, hipStream_t s) {
    const int tiles_m = int((M + BM - 1) / BM);
    const int total = plan.full + plan.split_tiles * plan.splits;
    const int64_t row_bytes = (K / block_values_of(QT)) * lay.stride;
    if (dots)
        hipLaunchKernelGGL((mmq_kernel<QT, BM, true>), dim3(total), dim3(256), 0, s, W, codes, xs, xsum, Y, dots,
                           partial, counters, int(M), int(N), int(K), row_bytes, lay.stride, lay.off, tiles_m,
                           plan.full, plan.split_tiles, plan.splits, plan.steps);
    else
        hipLaunchKernelGGL((mmq_kernel<QT, BM, false>), dim3(total), dim3(256), 0, s, W, codes, xs, xsum, Y, dots,
                           partial, counters, int(M), int(N), int(K), row_bytes, lay.stride, lay.off, tiles_m,
                           plan.full, plan.split_tiles, plan.splits, plan.steps);
    return hipGetLastError();
}

template <int QT>
hipError_t launch_typed(const uint8_t* W, const int8_t* codes, const float* xs, const int32_t* xsum,
                        float* Y, int32_t* dots, float* partial, unsigned* counters, int64_t M, int64_t N,
                        int64_t K, BlockLayout lay, hipStream_t s) {
    const MmqPlan plan = mmq_plan(QT, M, N, K);
    if (!counters && partial) {   // the caller's scratch: counters, then the partial tiles
        counters = reinterpret_cast<unsigned*>(partial);
        partial = reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(partial) + kSplitkCounterBytes);
    }
    if (plan.bm == 32)
        return launch_shaped<QT, 32>(W, codes, xs, xsum, Y, dots, partial, counters, M, N, K, lay, plan, s);
    return launch_shaped<QT, 128>(W, codes, xs, xsum, Y, dots, partial, counters, M, N, K, lay, plan, s);
}

}  // namespace

size_t mmq_smem_bytes(int type, int bm) {
    auto pick = [&](auto qt) -> size_t {
        constexpr int QT = decltype(qt)::value;
        return bm == 32 ? sizeof(Smem<QT, 32>) : bm == 128 ? sizeof(Smem<QT, 128>) : 0;
    };
    switch (type) {
        case kQ4_K: return pick(std::integral_constant<int, kQ4_K>{});
        case kQ5_K: return pick(std::integral_constant<int, kQ5_K>{});
        case kQ6_K: return pick(std::integral_constant<int, kQ6_K>{});
        case kQ8_0: return pick(std::integral_constant<int, kQ8_0>{});
        case kQ4_0: return pick(std::integral_constant<int, kQ4_0>{});
        case kQ4_1: return pick(std::integral_constant<int, kQ4_1>{});
        case kQ5_0: return pick(std::integral_constant<int, kQ5_0>{});
        case kQ5_1: return pick(std::integral_constant<int, kQ5_1>{});
        default: return 0;
    }
}

MmqPlan mmq_plan(int /*type*/, int64_t M, int64_t N, int64_t K) {
    // kTargetWorkgroups workgroups fill the chip.  Tiles are dealt whole while they fill it;
    // the tiles of a last, less than half full round (or all tiles, when there are fewer
    // than half a round of them) are cut into K ranges of at least kMinStepsPerSplit steps,
    // enough of them for half a round: one workgroup per CU.  (Ranges for a full round, two
    // per CU, were slower on nearly every shape timed: 7B ffn_up Q4_K 150.5 against 144.4 us,
    // Q8_0 144.2 against 136.2 us, 512 x 512 x 3584 16.4 against 15.4 us; the vocab head
    // at M = 9, whose last round then is not cut at all, 119.3 against 111.6 us.)  A function
    // of the shape alone, so the result does not depend on the device.
    MmqPlan p;
    // 128-row tiles while there are enough of them to fill more than half a round; else
    // (small M, or a small N) 32-row tiles, four times as many, so fewer are cut.
    const int64_t tiles128 = ((M + 127) / 128) * ((N + BN - 1) / BN);
    p.bm = M <= kSmallM || tiles128 * 2 <= kTargetWorkgroups ? 32 : 128;
    p.steps = int((K + KS - 1) / KS);
    const int64_t tiles = ((M + p.bm - 1) / p.bm) * ((N + BN - 1) / BN);
    const int64_t rem = tiles % kTargetWorkgroups;
    p.full = int(tiles);
    p.split_tiles = 0;
    p.splits = 1;
    if (rem > 0 && rem * 2 <= kTargetWorkgroups) {
        const int64_t splits = std::min<int64_t>(kTargetWorkgroups / 2 / rem, p.steps / kMinStepsPerSplit);
        if (splits >= 2) {
            p.full = int(tiles - rem);
            p.split_tiles = int(rem);
            p.splits = int(splits);
        }
    }
    return p;
}

size_t mmq_scratch_bytes(int type, int64_t M, int64_t N, int64_t K) {
    if (gemv_q8_applies(type, M, K) || mmq_kw_applies(type, BlockLayout{144, 0}, M, N, K)) return 0;
    const MmqPlan p = mmq_plan(type, M, N, K);
    return splitk_scratch_bytes(p.split_tiles, p.splits, int64_t(p.bm) * BN);
}

size_t mmq_partial_bytes(int type, int64_t M, int64_t N, int64_t K) {
    if (gemv_q8_applies(type, M, K) || mmq_kw_applies(type, BlockLayout{144, 0}, M, N, K)) return 0;
    const MmqPlan p = mmq_plan(type, M, N, K);
    return size_t(p.split_tiles) * size_t(p.splits) * size_t(p.bm) * BN * sizeof(float);
}

hipError_t launch_mmq(int type, BlockLayout lay, const uint8_t* W, const int8_t* codes, const float* xs,
                      const int32_t* xsum, float* Y, int32_t* dots, void* scratch, unsigned* counters, int64_t M,
                      int64_t N, int64_t K, hipStream_t s, const char** name) {
    if (gemv_q8_applies(type, M, K)) return launch_gemv_q8(type, lay, W, codes, xs, xsum, Y, dots, M, N, K, s, name);
    if (mmq_kw_applies(type, lay, M, N, K)) return launch_mmq_kw(W, codes, xs, xsum, Y, dots, M, N, K, s, name);
    float* partial = static_cast<float*>(scratch);
    const bool repacked = lay.off != 0 || (type == kQ6_K && lay.stride != 210);
    switch (type) {
        case kQ8_0:
            *name = repacked ? "mmq<q8_0 repacked>" : "mmq<q8_0>";
            return launch_typed<kQ8_0>(W, codes, xs, xsum, Y, dots, partial, counters, M, N, K, lay, s);
        case kQ4_K:
            *name = "mmq<q4_K>";
            return launch_typed<kQ4_K>(W, codes, xs, xsum, Y, dots, partial, counters, M, N, K, lay, s);
        case kQ6_K:
            *name = repacked ? "mmq<q6_K repacked>" : "mmq<q6_K>";
            return launch_typed<kQ6_K>(W, codes, xs, xsum, Y, dots, partial, counters, M, N, K, lay, s);
        case kQ5_K:
            *name = "mmq<q5_K>";
            return launch_typed<kQ5_K>(W, codes, xs, xsum, Y, dots, partial, counters, M, N, K, lay, s);
        case kQ4_0:
            *name = "mmq<q4_0>";
            return launch_typed<kQ4_0>(W, codes, xs, xsum, Y, dots, partial, counters, M, N, K, lay, s);
        case kQ4_1:
            *name = "mmq<q4_1>";
            return launch_typed<kQ4_1>(W, codes, xs, xsum, Y, dots, partial, counters, M, N, K, lay, s);
        case kQ5_0:
            *name = "mmq<q5_0>";
            return launch_typed<kQ5_0>(W, codes, xs, xsum, Y, dots, partial, counters, M, N, K, lay, s);
        case kQ5_1:
            *name = "mmq<q5_1>";
            return launch_typed<kQ5_1>(W, codes, xs, xsum, Y, dots, partial, counters, M, N, K, lay, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace mq
