// mq_gemm for Q4_K with M > 32 rows: the block dots on the fp8 matrix units.
//
// The product is the MMQ of "minfer CUDA Backend Design", 4.4 Execution dispatch
// (weights' block codes times an activation plane quantized to q8 blocks):
//
//   Y[m][n] = sum_b dx[m][b] * ( dw[n][b] * D[m][n][b] - mw[n][b] * S[m][b] ),
//   D[m][n][b] = sum_{i<32} c[n][32b+i] * q[m][32b+i]   (exact integers, |D| < 2^16)
//
// with dw = d * sc and mw = dmin * m the Q4_K sub-block factors, dx and S the
// activation block scale and code sum.
//
// Exact block dots in f32.  v_mfma_f32_32x32x64_f8f6f4 on OCP e4m3 operands multiplies
// e4m3 bytes 0..15 as the exact values p * 2^-9 (subnormals and the first binade share
// the spacing 2^-9), so a 4-bit weight code is already an e4m3 operand, and an 8-bit
// activation code is one as two digits, |q| = 16 h + l: the activation plane carries
// each block as [h of values 0..31 | l of values 0..31] (mq_quantize_act), and lane group
// g of the MFMA takes bytes 32g..32g+31 of the block's 64 bytes (the h digits for g = 0,
// the l digits for g = 1) against the block's 32 codes.  Each product then is exactly
// 2^-18 * c * q, and the MFMA returns D * 2^-18 in f32 with no rounding (every partial
// sum is an integer multiple of 2^-18 below 2^24 * 2^-18).  Compared with int8 block
// dots this saves the int32 -> f32 conversion of every element and block: the vector
// ALU does one fused multiply-add per element and block.
//
// Scales.  The element scale dx[m][b] * dw[n][b] * 2^18 comes from a bf16 matrix
// product with the f32 factors split into bf16 hi + lo terms (hi*hi + lo*hi + hi*lo,
// relative error below 2^-16), computed on the matrix units alongside the vector ALU of
// the other wave.  The min term sum_b (dx S)[m][b] * (-dmin m)[n][b] is a second bf16
// hi/lo product over the step's two blocks, accumulated straight into the output tile.
//
// Tiling.  One 512-thread workgroup (8 waves, 2 x 4) per CU owns a 128 x 256 tile of Y
// and walks its K range in steps of 64 values (2 blocks); each wave owns 2 x 2 MFMA
// tiles of 32 x 32.  Everything a step reads from memory -- the activation digit
// records (one 128-byte line per row) and scale records (contiguous per step), the
// weights' raw code bytes and super-block headers -- goes global -> LDS with
// buffer_load ... lds into a ring of three step slots, issued two steps ahead.  Eight
// lanes load one digit line, so each instruction reads whole cache lines.  Each lane
// then unpacks only bytes it loaded itself (weight nibbles to code bytes, headers to
// scale factors, scale records to the bf16 operand pairs of the scale products) into one
// of two work buffers, which needs no barrier; one workgroup barrier per step publishes
// the step.  Tiles that a last, partial round of workgroups would leave idle are cut
// into K ranges and summed in the same launch (mmq_splitk.h).
#include <algorithm>
#include <type_traits>

#include "mmq_splitk.h"
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

namespace {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int BM = 128;          // output tile rows (activation rows)
constexpr int BN = 256;          // output tile columns (weight rows)
constexpr int KS = 64;           // K values per step
constexpr int NB = KS / 32;      // blocks per step
constexpr int kWaves = 8;        // 2 (rows) x 4 (columns), each 64 x 64
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;
constexpr int kTargetWorkgroups = 256;   // one resident workgroup on each of 256 CUs
constexpr int kMinStepsPerSplit = 4;
constexpr int kBufferWord3 = 0x00020000;  // raw buffer resource: 32-bit data format, no swizzle
constexpr float kDotScale = 262144.0f;     // 2^18: D = MFMA result * 2^18

// Row (within a 32-row MFMA tile) of accumulator element v for lane group g.
__device__ __forceinline__ int acc_row(int v, int g) { return 8 * (v >> 2) + 4 * g + (v & 3); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kBufferWord3);
}

// x as bf16 hi = bf16(x) and lo = bf16(x - hi), packed hi | lo << 16.
__device__ __forceinline__ uint32_t bf16_hilo(float x) {
    const __bf16 hi = static_cast<__bf16>(x);
    const __bf16 lo = static_cast<__bf16>(x - static_cast<float>(hi));
    return uint32_t(__builtin_bit_cast(uint16_t, hi)) | (uint32_t(__builtin_bit_cast(uint16_t, lo)) << 16);
}

// Workgroup barrier after this wave's LDS writes are done.  (__syncthreads would also wait
// for every global load in flight -- its workgroup fence covers global memory -- and so
// drain the ring of loads issued steps ahead.)  The "memory" clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Wait until at most N vector memory operations of this wave are outstanding (the
// builtin, so that the compiler's own wait insertion knows about it).  gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima.
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One step's data as loaded from memory (global -> LDS directly).
//   A: the BM rows' 128-byte digit records, row-major; 16-byte chunk c of row r sits at
//      chunk position c ^ swz(r), swz(r) = (r / 2) % 8, so that the 16 lanes of a fragment
//      read (16 consecutive rows, one chunk) fall on 16 different bank groups;
//   ss: the BM rows' scale records (dx of blocks 0 and 1, code sum of blocks 0 and 1);
//   qs: weight code bytes qs[32c + 16h ..] of each row, chunk-major (chunk h of row n at
//      16 (h BN + n));
//   hdr: each weight row's super-block header (d, dmin, 12 scale bytes), row-major.
struct Slot {
    uint8_t A[BM * 128];
    uint8_t ss[BM * 16];
    uint8_t qs[BN * 32];
    uint8_t hdr[BN * 16];
};
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// One step's unpacked weight operand and the bf16 operand pairs of its scale products
// (8 bytes each: the two dwords one lane passes to v_mfma_f32_32x32x8_bf16; lane group g
// takes bf16 slots 4g..4g+3).
//   outer product dx (x) dw:  g = 0: A (dx_hi, dx_lo, 0, 0), B (dw_hi, dw_hi, 0, 0);
//                             g = 1: A (dx_hi, 0, 0, 0),     B (dw_lo, 0, 0, 0)
//   min term over the step's blocks (lane group g feeds block g):
//                             A (tx_hi, tx_hi, tx_lo, 0), B (mw_hi, mw_lo, mw_hi, 0)
struct Work {
    uint8_t B[BN * KS];         // weight codes, one e4m3 byte per value: chunk c = values 16 (c % 2).. of block c / 2
    uint2 dxq[2][NB * BM];      // [g][entry in the order of Slot::dx]
    uint2 dwq[2][NB][BN];       // [g][block][row]
    uint2 txq[NB * BM];         // dx * code sum, order of Slot::dx
    uint2 mwq[NB][BN];          // -dmin * m
};
static_assert(3 * sizeof(Slot) + 2 * sizeof(Work) <= 160 * 1024, "the ring fits the gfx950 LDS");

// Separate LDS arrays per ring position (compile-time indices): the compiler then waits
// for outstanding LDS-direct loads only before reads of the slot they write.
__shared__ __attribute__((aligned(16))) Slot g_slot0, g_slot1, g_slot2;
__shared__ __attribute__((aligned(16))) Work g_work0, g_work1;
template <int R> __device__ __forceinline__ Slot& slot_at() { return R == 0 ? g_slot0 : R == 1 ? g_slot1 : g_slot2; }
template <int R> __device__ __forceinline__ Work& work_at() { return R == 0 ? g_work0 : g_work1; }

// ------------------------------------------------------------------ loads of one step
// A step's loads (buffer_load ... lds, 1 KB per instruction), wave w taking:
//   digit lines: instructions w and w + 8 of 16, 8 rows each (8 lanes per 128-byte line);
//   weight code bytes: instruction w of 8 (32 rows x 2 lanes);
//   waves 0, 1: scale records of rows 64 w .. 64 w + 63;
//   waves 4..7: weight headers of rows 64 (w - 4) .. + 63.
// So waves 0, 1 and 4..7 issue 4 loads per step and waves 2, 3 issue 3.  The loads run
// two steps ahead; past the end of the K range they load the last step again (the
// copies are never read), which keeps the count the same for every step and every
// address inside the operands.  Rows past M or N read as zeros (out of the buffer
// ranges, checked on the per-lane offsets).
struct Loader {
    __amdgpu_buffer_rsrc_t ra, rs, rw;
    uint32_t voff_a[2];   // digit instructions wave, wave + 8
    uint32_t voff_q;      // code instruction
    uint32_t voff_x;      // scale record (waves 0, 1) or header (waves 4..7)
    int wave;
    int64_t step_stride;  // bytes between the same row's scale records of consecutive steps

    __device__ void init(const uint8_t* W, int64_t rb, const uint8_t* digits, const uint8_t* step_scales,
                         int m0, int n0, int M, int N, int K) {
        const int lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const int rows = min(BM, M - m0), wrows = min(BN, N - n0);
        const int T = (K + 63) / 64;
        ra = make_rsrc(digits + int64_t(m0) * T * 128, int64_t(rows) * T * 128);
        rs = make_rsrc(step_scales + int64_t(m0) * 16, (int64_t(T) * M - m0) * 16);
        rw = make_rsrc(W + int64_t(n0) * rb, int64_t(wrows) * rb);
        step_stride = int64_t(M) * 16;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = 8 * (wave + 8 * i) + lane / 8;         // row of this lane's LDS chunk
            const int c = (lane % 8) ^ swz(r);                    // the digit chunk that belongs there
            voff_a[i] = uint32_t(r * T * 128 + 16 * c);
        }
        {
            const int o = 1024 * wave + 16 * lane;               // LDS byte in Slot::qs
            const int h = o / (16 * BN), row = (o % (16 * BN)) / 16;
            voff_q = uint32_t(int64_t(row) * rb + 16 + 16 * h);
        }
        if (wave < 2)   // scale record of row 64 wave + lane (rows past M: out of range)
            voff_x = 64 * wave + lane < rows ? uint32_t((64 * wave + lane) * 16) : 0x80000000u;
        else
            voff_x = uint32_t(int64_t(64 * (wave - 4) + lane) * rb);  // header (waves 4..7)
    }

    template <int R>
    __device__ void issue(int k0) const {
        Slot& sl = slot_at<R>();
        const uint32_t t = uint32_t(k0 >> 6);
        const uint32_t wsoff = uint32_t(144 * (k0 >> 8) + 32 * ((k0 >> 6) & 3));   // super-block, 64-value chunk
#pragma unroll
        for (int i = 0; i < 2; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(sl.A + 1024 * (wave + 8 * i)), 16, voff_a[i],
                                                     t * 128, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(sl.qs + 1024 * wave), 16, voff_q, wsoff, 0, 0);
        if (wave < 2)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(sl.ss + 1024 * wave), 16, voff_x,
                                                     uint32_t(t * step_stride), 0, 0);
        else if (wave >= 4)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(sl.hdr + 1024 * (wave - 4)), 16, voff_x,
                                                     uint32_t(144 * (k0 >> 8)), 0, 0);
    }

    // wait for this wave's loads of the step before the most recently issued one
    __device__ void wait_previous() const {
        if (wave == 2 || wave == 3) vm_wait<3>();
        else vm_wait<4>();
    }
};

// Unpack the bytes this lane loaded for the step in slot R into work buffer WB (no
// barrier: a lane reads back only LDS bytes its own wave's loads wrote, once they have
// landed).
__device__ __forceinline__ uint2 pair(uint32_t a, uint32_t b) { return make_uint2(a, b); }

template <int R, int WB>
__device__ __forceinline__ void unpack(int k0) {
    const Slot& sl = slot_at<R>();
    Work& wk = work_at<WB>();
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    {   // codes: the lane's 16 bytes hold values 16h.. of sub-blocks 2c (low) and 2c + 1 (high nibbles)
        const int o = 1024 * wave + 16 * lane;
        const int h = o / (16 * BN), row = (o % (16 * BN)) / 16;
        const uint4 q = *reinterpret_cast<const uint4*>(sl.qs + o);
        const uint4 lo = make_uint4(q.x & 0x0F0F0F0Fu, q.y & 0x0F0F0F0Fu, q.z & 0x0F0F0F0Fu, q.w & 0x0F0F0F0Fu);
        const uint4 hi = make_uint4((q.x >> 4) & 0x0F0F0F0Fu, (q.y >> 4) & 0x0F0F0F0Fu, (q.z >> 4) & 0x0F0F0F0Fu,
                                    (q.w >> 4) & 0x0F0F0F0Fu);
        *reinterpret_cast<uint4*>(wk.B + h * (16 * BN) + 16 * row) = lo;            // block 0, values 16h..
        *reinterpret_cast<uint4*>(wk.B + (2 + h) * (16 * BN) + 16 * row) = hi;      // block 1, values 16h..
    }
    if (wave >= 4) {   // header of row 64 (wave - 4) + lane: factors of sub-blocks 2c and 2c + 1
        const int row = 64 * (wave - 4) + lane;
        const uint4 hd = *reinterpret_cast<const uint4*>(sl.hdr + 16 * row);
        const float d = half_bits_to_float(hd.x & 0xFFFFu);
        const float dmin = half_bits_to_float(hd.x >> 16);
        const int c = (k0 >> 6) & 3;
#pragma unroll
        for (int p = 0; p < NB; ++p) {
            uint32_t sc, mn;
            q4k_scale_min(hd.y, hd.z, hd.w, 2 * c + p, sc, mn);   // uniform branch: c is per step
            const uint32_t w = bf16_hilo(d * float(sc) * kDotScale);
            wk.dwq[0][p][row] = pair(__builtin_amdgcn_perm(w, w, 0x01000100u), 0u);
            wk.dwq[1][p][row] = pair(w >> 16, 0u);
            const uint32_t m = bf16_hilo(-(dmin * float(mn)));
            wk.mwq[p][row] = pair(m, m & 0xFFFFu);
        }
    } else if (wave < 2) {   // scale record of row 64 wave + lane: both blocks
        const int r = 64 * wave + lane;
        const uint4 sr = *reinterpret_cast<const uint4*>(sl.ss + 16 * r);
#pragma unroll
        for (int p = 0; p < NB; ++p) {
            const float dx = __uint_as_float(p ? sr.y : sr.x);
            const int32_t sum = int32_t(p ? sr.w : sr.z);
            const uint32_t x = bf16_hilo(dx);
            wk.dxq[0][p * BM + r] = pair(x, 0u);
            wk.dxq[1][p * BM + r] = pair(x & 0xFFFFu, 0u);
            const uint32_t tx = bf16_hilo(dx * float(sum));
            wk.txq[p * BM + r] = pair(__builtin_amdgcn_perm(tx, tx, 0x01000100u), tx >> 16);
        }
    }
}

// ------------------------------------------------------------------ kernel
template <bool DUMP>
__global__ __launch_bounds__(kThreads, 1) void mmq_f8_q4k_kernel(const uint8_t* __restrict__ W,
                                                                 const uint8_t* __restrict__ digits,
                                                                 const uint8_t* __restrict__ step_scales,
                                                                 float* __restrict__ Y, int32_t* __restrict__ dots,
                                                                 float* __restrict__ partial,
                                                                 unsigned* __restrict__ counters, int M, int N, int K,
                                                                 int64_t row_bytes, int tiles_m, int full,
                                                                 int split_tiles, int splits, int total_steps) {
    constexpr int TI = 2, TJ = 2;

    // Work split: workgroups [0, full) own whole tiles 0..full-1; the remaining split_tiles
    // tiles are each cut into `splits` K ranges, one workgroup per range.  Within each group
    // the ids are remapped so that the workgroups landing on one XCD take consecutive
    // logical ids, and consecutive ids are the M-tiles of one N-tile (the same weights).
    const int id = blockIdx.x;
    const bool whole = id < full;
    const int group = whole ? full : split_tiles * splits;
    const int j0 = whole ? id : id - full;
    const int jj = group % kXcds == 0 ? (j0 % kXcds) * (group / kXcds) + j0 / kXcds : j0;
    const int tile = whole ? jj : full + jj % split_tiles;
    const int piece = whole ? 0 : jj / split_tiles;
    const int pieces = whole ? 1 : splits;
    const int tm = tile % tiles_m, tn = tile / tiles_m;
    const int m0 = tm * BM, n0 = tn * BN;
    const int sbeg = int(int64_t(piece) * total_steps / pieces);
    const int nsteps = int(int64_t(piece + 1) * total_steps / pieces) - sbeg;
    const int kbeg = sbeg * KS;

    const int t = threadIdx.x;
    const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int g = lane >> 5, r32 = lane & 31;
    const int KB = K >> 5;

    v16f acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    Loader ld;
    ld.init(W, row_bytes, digits, step_scales, m0, n0, M, N, K);
    const int klast = kbeg + (nsteps - 1) * KS;   // the range's last step

    // One K-step on ring position R = s % 3 and work buffer WB = s % 2 (compile-time, so
    // every LDS address is a per-lane base plus an immediate and each slot is a separate LDS
    // array).  On entry the step's work buffer and digit records are complete and published
    // by the barrier; the loads of step s + 1 are in flight.
    auto step = [&](auto r_c, auto wb_c, int s) {
        constexpr int R = decltype(r_c)::value, WB = decltype(wb_c)::value;
        constexpr int R1 = (R + 1) % 3, R2 = (R + 2) % 3;
        const int k0 = kbeg + s * KS;
        ld.issue<R2>(min(k0 + 2 * KS, klast));   // slot R2 was last read by step s - 1

        const uint8_t* As = slot_at<R>().A;
        const Work& wk = work_at<WB>();
        const int arow0 = 64 * wm + r32;   // + 32 i
        const int brow0 = 64 * wn + r32;   // + 32 j

        // Products k = 4p + 2i + j (block p, tiles i, j): D (fp8 block dots) and S (scales).
        v8i a[TI], b[TJ];
        v4s oa[TI], ob[TJ];
        auto frags = [&](int p) {
#pragma unroll
            for (int i = 0; i < TI; ++i) {
                const int ar = arow0 + 32 * i;
                const v4i lo = *reinterpret_cast<const v4i*>(As + 128 * ar + 16 * ((4 * p + 2 * g) ^ swz(ar)));
                const v4i hi = *reinterpret_cast<const v4i*>(As + 128 * ar + 16 * ((4 * p + 2 * g + 1) ^ swz(ar)));
                a[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                oa[i] = __builtin_bit_cast(v4s, wk.dxq[g][p * BM + ar]);
            }
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                const int br = brow0 + 32 * j;
                const v4i lo = *reinterpret_cast<const v4i*>(wk.B + (2 * p) * (16 * BN) + 16 * br);
                const v4i hi = *reinterpret_cast<const v4i*>(wk.B + (2 * p + 1) * (16 * BN) + 16 * br);
                b[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                ob[j] = __builtin_bit_cast(v4s, wk.dwq[g][p][br]);
            }
        };
        auto products = [&](int i, int j, v16f& D, v16f& S) {
            const v16f z = {};
            D = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], z, 0, 0, 0, 0, 0, 0);
            S = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(oa[i], ob[j], z, 0, 0, 0);
        };
        auto consume = [&](int p, int i, int j, const v16f& D, const v16f& S) {
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = fmaf(D[v], S[v], acc[i][j][v]);
            asm volatile("" : "+v"(acc[i][j]));
            if constexpr (DUMP) {
                const int nn = n0 + brow0 + 32 * j;
                const int kb = (k0 >> 5) + p;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = m0 + 64 * wm + 32 * i + acc_row(v, g);
                    if (m < M && nn < N && kb < KB) dots[(int64_t(m) * N + nn) * KB + kb] = int(D[v] * kDotScale);
                }
            }
        };
        // min term of tile (i, j) for the step's 2 blocks: lane group g feeds block g
        auto min_term = [&](int i, int j) {
            const int ar = arow0 + 32 * i, br = brow0 + 32 * j;
            const v4s ma = __builtin_bit_cast(v4s, wk.txq[g * BM + ar]);
            const v4s mb = __builtin_bit_cast(v4s, wk.mwq[g][br]);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(ma, mb, acc[i][j], 0, 0, 0);
        };

        v16f D[2], S[2];
#pragma unroll
        for (int p = 0; p < NB; ++p) {
            frags(p);
            products(0, 0, D[0], S[0]);
#pragma unroll
            for (int k = 0; k < TI * TJ; ++k) {
                const int i = k / TJ, j = k % TJ;
                if (k + 1 < TI * TJ) products((k + 1) / TJ, (k + 1) % TJ, D[(k + 1) & 1], S[(k + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
                consume(p, i, j, D[k & 1], S[k & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j) min_term(i, j);

        // the next step's data: this wave's loads of step s + 1 have landed; unpack them
        if (s + 1 < nsteps) {
            // (the block-dot export's stores count in vmcnt too: it waits for everything)
            if constexpr (DUMP) vm_wait<0>();
            else ld.wait_previous();
            unpack<R1, WB ^ 1>(k0 + KS);
        }
        lds_barrier();   // step s + 1 is published (every wave waited for its own loads); slot R is free
    };

    // prologue: steps 0 and 1 in flight, step 0 unpacked and published
    ld.issue<0>(kbeg);
    ld.issue<1>(min(kbeg + KS, klast));
    ld.wait_previous();
    unpack<0, 0>(kbeg);
    lds_barrier();

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    for (int s = 0;;) {
        step(I0{}, I0{}, s);
        if (++s >= nsteps) break;
        step(I1{}, I1{}, s);
        if (++s >= nsteps) break;
        step(I2{}, I0{}, s);
        if (++s >= nsteps) break;
        step(I0{}, I1{}, s);
        if (++s >= nsteps) break;
        step(I1{}, I0{}, s);
        if (++s >= nsteps) break;
        step(I2{}, I1{}, s);
        if (++s >= nsteps) break;
    }
    vm_wait<0>();   // no LDS-direct load of the ring may land after the workgroup ends

    if constexpr (DUMP) return;
    // A split tile puts its partial into its piece's slot, and the piece that counts in
    // last sums all pieces' slots in piece order into Y.
    float* tile_slots = whole ? nullptr : partial + size_t(tile - full) * size_t(pieces) * (BM * BN);
    float* my_slot = whole ? nullptr : tile_slots + size_t(piece) * (BM * BN);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int n = n0 + 64 * wn + 32 * j + r32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + 64 * wm + 32 * i + acc_row(v, g);
                if (!whole)
                    splitk_put(my_slot, splitk_index<TI, TJ, kThreads>(i, j, v, t), acc[i][j][v]);
                else if (m < M && n < N)
                    Y[int64_t(m) * N + n] = acc[i][j][v];
            }
        }
    if (whole || !splitk_arrive(counters + (tile - full), pieces, reinterpret_cast<unsigned*>(&g_slot0))) return;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            float y[16];
            splitk_sum_tile<TI, TJ, kThreads>(tile_slots, pieces, i, j, y);
            const int n = n0 + 64 * wn + 32 * j + r32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + 64 * wm + 32 * i + acc_row(v, g);
                if (m < M && n < N) Y[int64_t(m) * N + n] = y[v];
            }
        }
}

template __global__ void mmq_f8_q4k_kernel<false>(const uint8_t* __restrict__, const uint8_t* __restrict__,
                                                  const uint8_t* __restrict__,
                                                  float* __restrict__, int32_t* __restrict__, float* __restrict__,
                                                  unsigned* __restrict__, int, int, int, int64_t, int, int, int, int,
                                                  int);
template __global__ void mmq_f8_q4k_kernel<true>(const uint8_t* __restrict__, const uint8_t* __restrict__,
                                                 const uint8_t* __restrict__,
                                                 float* __restrict__, int32_t* __restrict__, float* __restrict__,
                                                 unsigned* __restrict__, int, int, int, int64_t, int, int, int, int,
                                                 int);

}  // namespace

// Q4_K products with at least one whole round of output tiles.  Smaller products (fewer
// tiles than workgroups, e.g. 512 x 3584 or 512 x 512) run faster on the int8 kernel, whose
// smaller tiles and separate K-split sum fill the chip with less per-tile overhead.
bool mmq_f8_applies(int type, int64_t M, int64_t N) {
    return type == kQ4_K && M > 32 && ((M + BM - 1) / BM) * ((N + BN - 1) / BN) >= kTargetWorkgroups;
}

MmqPlan mmq_f8_plan(int64_t M, int64_t N, int64_t K) {
    // As mmq_plan, with 64-value K-steps: tiles are dealt whole while they fill rounds of
    // kTargetWorkgroups; the tiles of a last round that is at most half full (or all tiles,
    // when there are fewer than half a round) are cut into K ranges of at least
    // kMinStepsPerSplit steps, enough to fill that round.  A function of the shape alone.
    MmqPlan p;
    p.bm = BM;
    p.steps = int((K + KS - 1) / KS);
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    const int64_t rem = tiles % kTargetWorkgroups;
    p.full = int(tiles);
    p.split_tiles = 0;
    p.splits = 1;
    if (rem > 0 && rem * 2 <= kTargetWorkgroups) {
        const int64_t splits = std::min<int64_t>(kTargetWorkgroups / rem, p.steps / kMinStepsPerSplit);
        if (splits >= 2) {
            p.full = int(tiles - rem);
            p.split_tiles = int(rem);
            p.splits = int(splits);
        }
    }
    return p;
}

size_t mmq_f8_scratch_bytes(int64_t M, int64_t N, int64_t K) {
    const MmqPlan p = mmq_f8_plan(M, N, K);
    return splitk_scratch_bytes(p.split_tiles, p.splits, int64_t(BM) * BN);
}

size_t mmq_f8_partial_bytes(int64_t M, int64_t N, int64_t K) {
    const MmqPlan p = mmq_f8_plan(M, N, K);
    return size_t(p.split_tiles) * size_t(p.splits) * size_t(BM) * BN * sizeof(float);
}

hipError_t launch_mmq_f8(int type, const uint8_t* W, const uint8_t* digits, const uint8_t* step_scales, float* Y,
                         int32_t* dots, void* scratch, unsigned* counters, int64_t M, int64_t N, int64_t K,
                         hipStream_t s, const char** name) {
    if (type != kQ4_K) return hipErrorInvalidValue;
    *name = "mmq_f8<q4_K>";
    const MmqPlan plan = mmq_f8_plan(M, N, K);
    const int tiles_m = int((M + BM - 1) / BM);
    const int total = plan.full + plan.split_tiles * plan.splits;
    const int64_t row_bytes = (K / 256) * 144;
    float* partial = static_cast<float*>(scratch);
    if (!counters && scratch)
        counters = reinterpret_cast<unsigned*>(static_cast<uint8_t*>(scratch) +
                                               splitk_counter_offset(plan.split_tiles, plan.splits, int64_t(BM) * BN));
    if (dots)
        hipLaunchKernelGGL(mmq_f8_q4k_kernel<true>, dim3(total), dim3(kThreads), 0, s, W, digits, step_scales, Y, dots,
                           partial, counters, int(M), int(N), int(K), row_bytes, tiles_m, plan.full,
                           plan.split_tiles, plan.splits, plan.steps);
    else
        hipLaunchKernelGGL(mmq_f8_q4k_kernel<false>, dim3(total), dim3(kThreads), 0, s, W, digits, step_scales, Y, dots,
                           partial, counters, int(M), int(N), int(K), row_bytes, tiles_m, plan.full,
                           plan.split_tiles, plan.splits, plan.steps);
    return hipGetLastError();
}

}  // namespace mq
