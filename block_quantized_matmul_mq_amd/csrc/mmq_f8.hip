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
#include <cstddef>
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
// builtin: the compiler keeps it as written).  gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima.
template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// buffer_load_dwordx4 ... lds: 16 bytes per lane from buffer offset voff + soff to LDS
// bytes lds + 16 lane.  Written as asm so that the compiler does not track these loads:
// it would otherwise wait for some of them before every read of any ring slot (its alias
// tracking of LDS-direct loads does not separate the slots), while the ring's own
// protocol -- every wave waits for its own loads of a step, then the workgroup barrier --
// already orders them.  The load has no destination register; M0 (which nothing else in
// the kernel uses) carries the LDS address and needs one wait state before the load.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory");
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
// LDS byte address of byte `off` of ring slot R (a constant plus `off`).
template <int R> __device__ __forceinline__ uint32_t slot_lds(uint32_t off) {
    return uint32_t(uintptr_t((const lds_void*)&slot_at<R>())) + off;
}

// ------------------------------------------------------------------ loads of one step
// A step's loads (buffer_load ... lds, 1 KB per instruction), wave w taking:
//   digit lines: instructions w and w + 8 of 16, 8 rows each (8 lanes per 128-byte line);
//   weight code bytes: instruction w of 8 (32 rows x 2 lanes);
//   waves 0..3: scale records of rows 64 (w % 2) .. + 63 (waves 2 and 3 load the same
//     bytes as waves 0 and 1 into the same place);
//   waves 4..7: weight headers of rows 64 (w - 4) .. + 63.
// Every wave issues the same 4 loads per step (only their operands differ), so the wait
// for a step's loads is one count for every wave and the compiler sees that a slot's
// loads are complete once that wait and the barrier after it have passed.  The loads run
// two steps ahead; past the end of the K range they load the last step again (the copies
// are never read), which keeps every address inside the operands.  Rows past M or N read
// as zeros (out of the buffer ranges, checked on the per-lane offsets).
struct Loader {
    __amdgpu_buffer_rsrc_t ra, rx, rw;
    uint32_t voff_a[2];   // digit instructions wave, wave + 8
    uint32_t voff_q;      // code instruction
    uint32_t voff_x;      // scale record (waves 0..3) or header (waves 4..7)
    int wave;
    bool scales;          // this wave's fourth load is a scale record (else a header)
    int64_t step_stride;  // bytes between the same row's scale records of consecutive steps

    __device__ void init(const uint8_t* W, int64_t rb, const uint8_t* digits, const uint8_t* step_scales,
                         int m0, int n0, int M, int N, int K) {
        const int lane = threadIdx.x & 63;
        wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        scales = wave < 4;
        const int rows = min(BM, M - m0), wrows = min(BN, N - n0);
        const int T = (K + 63) / 64;
        ra = make_rsrc(digits + int64_t(m0) * T * 128, int64_t(rows) * T * 128);
        rw = make_rsrc(W + int64_t(n0) * rb, int64_t(wrows) * rb);
        rx = scales ? make_rsrc(step_scales + int64_t(m0) * 16, (int64_t(T) * M - m0) * 16) : rw;
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
        if (scales) {   // scale record of row 64 (wave % 2) + lane (rows past M: out of range)
            const int r = 64 * (wave & 1) + lane;
            voff_x = r < rows ? uint32_t(r * 16) : 0x80000000u;
        } else {
            voff_x = uint32_t(int64_t(64 * (wave - 4) + lane) * rb);  // header
        }
    }

    // Load PART (0, 1: digit lines; 2: code bytes; 3: scale record or header) of the step
    // at k0 into slot R.
    template <int R, int PART>
    __device__ void issue_part(int k0) const {
        const uint32_t t = uint32_t(k0 >> 6);
        if constexpr (PART < 2) {
            dma16(ra, slot_lds<R>(offsetof(Slot, A) + 1024 * (wave + 8 * PART)), voff_a[PART], t * 128);
        } else if constexpr (PART == 2) {   // super-block, 64-value chunk
            dma16(rw, slot_lds<R>(offsetof(Slot, qs) + 1024 * wave), voff_q,
                  uint32_t(144 * (k0 >> 8) + 32 * ((k0 >> 6) & 3)));
        } else {
            const uint32_t xdst =
                scales ? offsetof(Slot, ss) + 1024 * (wave & 1) : offsetof(Slot, hdr) + 1024 * (wave - 4);
            dma16(rx, slot_lds<R>(xdst), voff_x, scales ? uint32_t(t * step_stride) : uint32_t(144 * (k0 >> 8)));
        }
    }
    template <int R>
    __device__ void issue(int k0) const {
        issue_part<R, 0>(k0);
        issue_part<R, 1>(k0);
        issue_part<R, 2>(k0);
        issue_part<R, 3>(k0);
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
        // The loads of step s + 2 go to slot R2 (last read in step s - 1), issued in four
        // parts spread over the products so that the waves' loads reach the memory pipeline
        // a few at a time.
        const int k2 = min(k0 + 2 * KS, klast);
        ld.issue_part<R2, 0>(k2);

        // The next step's data: once this wave's loads of step s + 1 have landed (at most
        // `newer` loads issued after them outstanding), unpack them (work buffer WB ^ 1 was
        // last read in step s - 1).  The two waves that share a SIMD (wm = 0 and wm = 1) do
        // this at different points of the step, so that one wave's unpacking (vector ALU and
        // LDS) runs beside the other's matrix products.
        auto unpack_next = [&](auto newer_c) {
            if (s + 1 < nsteps) {
                // (the block-dot export's stores count in vmcnt too: it waits for everything)
                if constexpr (DUMP) vm_wait<0>();
                else vm_wait<decltype(newer_c)::value>();
                unpack<R1, WB ^ 1>(k0 + KS);
            }
        };

        const uint8_t* As = slot_at<R>().A;
        const Work& wk = work_at<WB>();
        const int arow0 = 64 * wm + r32;   // + 32 i
        const int brow0 = 64 * wn + r32;   // + 32 j

        // Products kk = 4p + 2i + j (block p, tiles i, j): D (fp8 block dots) and S (scales).
        // Operands load one at a time, so that block 1's load into the registers of block
        // 0's as soon as their last product has been issued.
        v8i a[TI], b[TJ];
        v4s oa[TI], ob[TJ];
        auto load_a = [&](int p, int i) {
            const int ar = arow0 + 32 * i;
            const v4i lo = *reinterpret_cast<const v4i*>(As + 128 * ar + 16 * ((4 * p + 2 * g) ^ swz(ar)));
            const v4i hi = *reinterpret_cast<const v4i*>(As + 128 * ar + 16 * ((4 * p + 2 * g + 1) ^ swz(ar)));
            a[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            oa[i] = __builtin_bit_cast(v4s, wk.dxq[g][p * BM + ar]);
        };
        auto load_b = [&](int p, int j) {
            const int br = brow0 + 32 * j;
            const v4i lo = *reinterpret_cast<const v4i*>(wk.B + (2 * p) * (16 * BN) + 16 * br);
            const v4i hi = *reinterpret_cast<const v4i*>(wk.B + (2 * p + 1) * (16 * BN) + 16 * br);
            b[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            ob[j] = __builtin_bit_cast(v4s, wk.dwq[g][p][br]);
        };
        // The short scale product first: the wave then waits at most its 32 cycles before
        // the block dot (64 cycles) issues, and the previous product's 16 FMAs run beside
        // the block dot.
        auto products = [&](int i, int j, v16f& D, v16f& S) {
            const v16f z = {};
            S = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(oa[i], ob[j], z, 0, 0, 0);
            D = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], z, 0, 0, 0, 0, 0, 0);
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

        // The min term first: its products run while the first operands load.
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j) min_term(i, j);
        load_a(0, 0);
        load_b(0, 0);
        load_b(0, 1);
        load_a(0, 1);

        static_assert(TI == 2 && TJ == 2 && NB == 2, "the operand schedule below is written for 2 x 2 tiles");
        v16f D[2], S[2];
        products(0, 0, D[0], S[0]);
#pragma unroll
        for (int kk = 0; kk < NB * TI * TJ; ++kk) {
            const int p = kk / (TI * TJ), i = (kk / TJ) % TI, j = kk % TJ;
            const int kn = kk + 1;
            if (kn < NB * TI * TJ) products((kn / TJ) % TI, kn % TJ, D[kn & 1], S[kn & 1]);
            __builtin_amdgcn_sched_barrier(0);
            consume(p, i, j, D[kk & 1], S[kk & 1]);
            __builtin_amdgcn_sched_barrier(0);
            // block 1's operands, each once the products of block 0 that read its
            // registers have been issued (a0 by product 1, b0 by 2, a1 and b1 by 3)
            if (kk == 0) load_a(1, 0);
            if (kk == 1) {
                load_b(1, 0);
                ld.issue_part<R2, 1>(k2);
            }
            if (kk == 2) {
                load_b(1, 1);
                load_a(1, 1);
            }
            if (kk == 3) {
                ld.issue_part<R2, 2>(k2);
                if (wm == 1) unpack_next(std::integral_constant<int, 3>{});
            }
            if (kk == 5) ld.issue_part<R2, 3>(k2);
        }

        if (wm == 0) unpack_next(std::integral_constant<int, 4>{});
        lds_barrier();   // step s + 1 is published (every wave waited for its own loads); slot R is free
    };

    // prologue: steps 0 and 1 in flight, step 0 unpacked and published
    ld.issue<0>(kbeg);
    ld.issue<1>(min(kbeg + KS, klast));
    vm_wait<4>();
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
    if (whole) {
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j) {
                const int n = n0 + 64 * wn + 32 * j + r32;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = m0 + 64 * wm + 32 * i + acc_row(v, g);
                    if (m < M && n < N) Y[int64_t(m) * N + n] = acc[i][j][v];
                }
            }
        return;
    }
    constexpr uint32_t kSlotBytes = BM * BN * sizeof(float);
    const __amdgpu_buffer_rsrc_t slots =
        make_rsrc(partial + size_t(tile - full) * size_t(pieces) * (BM * BN), int64_t(pieces) * kSlotBytes);
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; v += 4)
                splitk_put<kThreads>(slots, uint32_t(piece) * kSlotBytes, ((i * TJ + j) * 16 + v) / 4,
                                     splitk_f4{acc[i][j][v], acc[i][j][v + 1], acc[i][j][v + 2], acc[i][j][v + 3]});
    if (!splitk_arrive(counters + (tile - full), pieces, reinterpret_cast<unsigned*>(&g_slot0))) return;
#pragma unroll
    for (int i = 0; i < TI; ++i) {   // one row of accumulator tiles at a time (registers)
        float y[TJ * 16];
        splitk_sum<TJ * 16, kThreads>(slots, kSlotBytes, pieces, i * TJ * 4, y);
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int n = n0 + 64 * wn + 32 * j + r32;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int m = m0 + 64 * wm + 32 * i + acc_row(v, g);
                if (m < M && n < N) Y[int64_t(m) * N + n] = y[j * 16 + v];
            }
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

size_t mmq_f8_lds_bytes() { return 3 * sizeof(Slot) + 2 * sizeof(Work); }

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
