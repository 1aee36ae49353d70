// mq_gemm for Q4_K weights in the MMQ plane that mq_repack writes: the block dots on the
// fp6 matrix units.
//
// The product is the MMQ of "minfer CUDA Backend Design", 4.4 Execution dispatch (weights'
// block codes times an activation plane quantized to q8 blocks), over the pre-decoded
// weight plane of the same page, 2.3 Weight residency and registry:
//
//   Y[m][n] = sum_b dx[m][b] * ( dw[n][b] * D[m][n][b] - dmin m[n][b] * S[m][b] ),
//   D[m][n][b] = sum_{i<32} c[n][32b+i] * q[m][32b+i]   (exact integers)
//
// with dw = d * sc and dmin m the Q4_K sub-block factors, dx and S the activation block
// scale and code sum.
//
// Exact block dots in f32.  OCP FP6 E2M3 holds every multiple of 1/2 from -7.5 to 7.5
// exactly, so the plane stores a 4-bit weight code c as the E2M3 code of c / 2, and the
// activation plane stores a code q = 16 h + l (h = q >> 4 in -8..7, l = q & 15) as the
// E2M3 codes of h / 2 and of l / 2.  v_mfma_scale_f32_32x32x64_f8f6f4 takes the block's
// h digits in K-slots 0..31 (lane group 0, block scale 2^5) and its l digits in K-slots
// 32..63 (lane group 1, block scale 2^1) against the block's weight codes in both halves:
// sum_j (16 h_j + l_j) c_j / 2 = D / 2, every partial sum a multiple of 1/2 below 2^15, so
// the f32 result is D / 2 with no rounding.  At the fp6 rate this MFMA costs what one int8
// 32x32x32 block dot costs, and it returns f32: the vector ALU does one fused multiply-add
// per element and block.
//
// Scales.  The element scale 2 dx[m][b] * dw[n][b] comes from a bf16 matrix product of the
// factors' hi + lo parts (each lane group multiplies out (x_hi + x_lo)(y_hi + y_lo), and
// there are two; relative error below 2^-16), on the matrix units; the min term
// sum_b (dx S)[m][b] * (-dmin m)[n][b] is a second bf16 hi/lo product over the step's two
// blocks (lane group g takes block g), accumulated straight into the output tile.  Both
// planes carry these bf16 operands ready made, so the kernel does no unpacking at all.
//
// Tiling.  A 256-thread workgroup (4 waves, 2 x 2), two resident per CU, owns a 128 x 128
// tile of Y and walks its K range in steps of 64 values (2 blocks); each wave owns 2 x 2
// MFMA tiles of 32 x 32.  A step's operands are 16 KB of the activation plane (its 128
// rows) and 10 KB of the weight plane (its 128 rows), each a few contiguous pieces in memory
// that go global -> LDS with buffer_load ... lds into a ring of three step slots (79 KB, so
// two rings fit a CU), issued two steps ahead; one workgroup barrier per step publishes a
// slot, placed before the step's last burst of products so that the next step's first
// operand reads run under its multiply-adds.  The two workgroups of a CU keep separate
// barriers, so one's waits overlap the other's products.  Tiles that a last, partial round
// of workgroups would leave idle are cut into K ranges and summed in the same launch
// (mmq_splitk.h).
#include <algorithm>
#include <cstddef>
#include <type_traits>

#include "mmq_common.h"
#include "mmq_splitk.h"
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((ext_vector_type(4)));

constexpr int BM = kF6TileRows;   // output tile rows (activation rows), 128
constexpr int BN = 128;           // output tile columns (weight rows)
constexpr int KS = 64;            // K values per step (two blocks)
constexpr int kWaves = 4;         // 2 (rows) x 2 (columns), each 64 x 64
constexpr int kThreads = 64 * kWaves;
constexpr int kXcds = 8;
constexpr int kTargetWorkgroups = 512;   // two resident workgroups on each of 256 CUs
constexpr int kMinStepsPerSplit = 4;
constexpr int kScaleH = 127 + 5;   // E8M0 2^5: block scale of the h / 2 digits
constexpr int kScaleL = 127 + 1;   // E8M0 2^1: block scale of the l / 2 digits
constexpr int kScaleOne = 127;     // E8M0 2^0
constexpr int kFmtE2M3 = 2;        // f8f6f4 operand format code of FP6 E2M3

// One step's operands in LDS, byte for byte the pieces of the two planes (mq_internal.h):
//   a16 [2u + g][row]  bytes 0..15 of the fp6 record of block u's h (g = 0) or l (g = 1) digits
//   a8  [2u + g][row]  bytes 16..23 of it
//   ao  [u][row]       dx operand pair (dx_hi | dx_lo << 16) twice
//   am  [u][row]       min-term operand pair (tx_hi | tx_hi << 16, tx_lo | tx_lo << 16), tx = dx S
//   b16 [u][row]       bytes 0..15 of the fp6 record of block u's weight codes
//   b8  [u][row]       bytes 16..23 of it
//   bo  [u][row]       dw operand pair (dw_hi | dw_hi << 16, dw_lo | dw_lo << 16)
//   bm  [u][row]       min-term operand pair (mw_hi | mw_lo << 16) twice, mw = -dmin m
// Every MFMA operand read below is 32 (or 16) lanes on consecutive rows of one array: no
// LDS bank conflicts.
struct Slot {
    uint8_t a16[4][BM][16];
    uint8_t a8[4][BM][8];
    uint8_t ao[2][BM][8];
    uint8_t am[2][BM][8];
    uint8_t b16[2][BN][16];
    uint8_t b8[2][BN][8];
    uint8_t bo[2][BN][8];
    uint8_t bm[2][BN][8];
};
static_assert(sizeof(Slot) == 26 * 1024, "a step slot is 26 loads of 1 KB");
static_assert(offsetof(Slot, b16) == 16 * 1024, "activation part first, 16 KB");
static_assert(3 * sizeof(Slot) + 1024 <= 80 * 1024, "two rings fit the gfx950 LDS");

__shared__ __attribute__((aligned(16))) Slot g_slot0, g_slot1, g_slot2;
__shared__ __attribute__((aligned(16))) uint8_t g_sink[1024];   // target of the loads that carry nothing
template <int R> __device__ __forceinline__ Slot& slot_at() { return R == 0 ? g_slot0 : R == 1 ? g_slot1 : g_slot2; }
template <int R> __device__ __forceinline__ uint32_t slot_lds(uint32_t off) {
    return uint32_t(uintptr_t((const __attribute__((address_space(3))) void*)&slot_at<R>())) + off;
}

// Byte offset, inside one step's slab of the activation plane (R = padded rows), of load
// i (0..15) of the workgroup whose rows start at m0: loads 1024 i .. of the slot's
// activation part.
__device__ __forceinline__ uint32_t act_piece(int i, int R, int m0) {
    if (i < 8) return uint32_t((i >> 1) * 16 * R + 16 * m0 + 1024 * (i & 1));   // a16[2u + g]
    if (i < 12) return uint32_t(64 * R + (i - 8) * 8 * R + 8 * m0);             // a8[2u + g]
    if (i < 14) return uint32_t(96 * R + (i - 12) * 8 * R + 8 * m0);            // ao[u]
    return uint32_t(112 * R + (i - 14) * 8 * R + 8 * m0);                        // am[u]
}
// The same for load j (0..19) of the weight part (R = padded weight rows, n0 the tile's
// first row): b16 4 loads per block, b8 / bo / bm 2 loads per block.
__device__ __forceinline__ uint32_t weight_piece(int j, int R, int n0) {
    if (j < 4) return uint32_t((j >> 1) * 16 * R + 16 * n0 + 1024 * (j & 1));
    const int sec = (j - 4) >> 1, u = (j - 4) & 1;   // b8, bo, bm
    return uint32_t((32 + 16 * sec) * R + u * 8 * R + 8 * n0);
}

// ------------------------------------------------------------------ kernel
template <bool DUMP>
__global__ __launch_bounds__(kThreads, 2) void mmq_f6_q4k_kernel(const uint8_t* __restrict__ Wp,
                                                                 const uint8_t* __restrict__ Ap,
                                                                 float* __restrict__ Y, int32_t* __restrict__ dots,
                                                                 float* __restrict__ partial,
                                                                 unsigned* __restrict__ counters, int M, int N, int K,
                                                                 int Mp, int Np, int tiles_m, int full,
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

    const int t = threadIdx.x;
    const int lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int g = lane >> 5, r32 = lane & 31;
    const int KB = K >> 5;
    const int a_slab = 128 * Mp, w_slab = 80 * Np;   // bytes of one step of each plane

    v16f acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // This wave's loads of a step: loads wave + 4 k (k = 0..6) of the step's 26 (16 of the
    // activation part, then 10 of the weight part).  Each lane moves 16 bytes at offset
    // piece + 16 lane of the step's slab: the piece offset (uniform) goes in soffset, the
    // lane's column in voffset.  Waves 2 and 3 have no seventh load: theirs reads past the
    // buffer (voffset 2^31: zeros, no memory traffic) into an LDS sink, so that every wave
    // issues the same count and the step has no branch.
    uint32_t spiece[7];
#pragma unroll
    for (int k = 0; k < 7; ++k) {
        const int i = wave + 4 * k;
        spiece[k] = i < 16 ? act_piece(i, Mp, m0) : i < 26 ? weight_piece(i - 16, Np, n0) : 0u;
    }
    const uint32_t vlane = 16 * lane;
    const uint32_t vlast = wave + 24 < 26 ? vlane : 0x80000000u;
    const uint32_t sink_lds = uint32_t(uintptr_t((const __attribute__((address_space(3))) void*)&g_sink));
    const int tlast = sbeg + nsteps - 1;
    auto issue = [&](auto r_c, auto k_c, int ts) {
        constexpr int R = decltype(r_c)::value, k = decltype(k_c)::value;
        const int i = wave + 4 * k;
        if constexpr (k < 4) {
            lds_dma16(raw_rsrc(Ap + int64_t(ts) * a_slab, a_slab), slot_lds<R>(1024 * i), vlane, spiece[k]);
        } else {
            const uint32_t dst = k < 6 || i < 26 ? slot_lds<R>(1024 * i) : sink_lds;
            lds_dma16(raw_rsrc(Wp + int64_t(ts) * w_slab, w_slab), dst, k < 6 ? vlane : vlast, spiece[k]);
        }
    };
    auto issue_all = [&](auto r_c, int ts) {
        issue(r_c, std::integral_constant<int, 0>{}, ts);
        issue(r_c, std::integral_constant<int, 1>{}, ts);
        issue(r_c, std::integral_constant<int, 2>{}, ts);
        issue(r_c, std::integral_constant<int, 3>{}, ts);
        issue(r_c, std::integral_constant<int, 4>{}, ts);
        issue(r_c, std::integral_constant<int, 5>{}, ts);
        issue(r_c, std::integral_constant<int, 6>{}, ts);
    };

    const int scale_a = g ? kScaleL : kScaleH;
    const int arow0 = 64 * wm + r32;   // + 32 i
    const int brow0 = 64 * wn + r32;   // + 32 j

    // Operands of block u of a step: the activation digits and dx pair of tiles i, the
    // weight codes and dw pair of tiles j; and the min-term pairs of the step's two blocks
    // (lane group g reads block g).
    struct Ops {
        v8i a[TI], b[TJ];
        v4s oa[TI], ob[TJ];
    };
    struct MinOps {
        v4s ma[TI], mb[TJ];
    };
    auto load_ops = [&](const Slot& sl, int u, Ops& o) {
#pragma unroll
        for (int i = 0; i < TI; ++i) {
            const int r = arow0 + 32 * i;
            const uint4 p = *reinterpret_cast<const uint4*>(sl.a16[2 * u + g][r]);
            const uint2 q = *reinterpret_cast<const uint2*>(sl.a8[2 * u + g][r]);
            o.a[i] = v8i{int(p.x), int(p.y), int(p.z), int(p.w), int(q.x), int(q.y), 0, 0};
            o.oa[i] = *reinterpret_cast<const v4s*>(sl.ao[u][r]);
        }
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int r = brow0 + 32 * j;
            const uint4 p = *reinterpret_cast<const uint4*>(sl.b16[u][r]);
            const uint2 q = *reinterpret_cast<const uint2*>(sl.b8[u][r]);
            o.b[j] = v8i{int(p.x), int(p.y), int(p.z), int(p.w), int(q.x), int(q.y), 0, 0};
            o.ob[j] = *reinterpret_cast<const v4s*>(sl.bo[u][r]);
        }
    };
    auto load_min = [&](const Slot& sl, MinOps& mo) {
#pragma unroll
        for (int i = 0; i < TI; ++i) mo.ma[i] = *reinterpret_cast<const v4s*>(sl.am[g][arow0 + 32 * i]);
#pragma unroll
        for (int j = 0; j < TJ; ++j) mo.mb[j] = *reinterpret_cast<const v4s*>(sl.bm[g][brow0 + 32 * j]);
    };

    Ops cur0, cur1;   // block 0 and block 1 operands of the current step
    MinOps mins;

    // Product p = 4 u + 2 i + j of a step is tile (i, j) of block u: its scale product S
    // and block dot D (two MFMAs), then 16 multiply-adds acc[i][j] += D * S.  The products
    // are software-pipelined by one: the two MFMAs of product p are issued each followed by
    // 8 of product p - 1's multiply-adds, so a wave's own stream keeps the matrix core and
    // the vector ALU busy together whatever the other wave on the SIMD is doing.  The step is
    // a single basic block; sched_group_barrier fixes the interleave.
    v16f S[2], D[2];
    auto mfma_s = [&](const Ops& o, int i, int j, v16f& out) {
        out = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(o.oa[i], o.ob[j], v16f{}, 0, 0, 0);
    };
    auto mfma_d = [&](const Ops& o, int i, int j, v16f& out) {
        out = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(o.a[i], o.b[j], v16f{}, kFmtE2M3, kFmtE2M3, 0, scale_a,
                                                              0, kScaleOne);
    };
    auto fmas = [&](int p, int half, int ts) {
        const int i = (p >> 1) & 1, j = p & 1, buf = p & 1;
#pragma unroll
        for (int v = 8 * half; v < 8 * half + 8; ++v) acc[i][j][v] = fmaf(D[buf][v], S[buf][v], acc[i][j][v]);
        if constexpr (DUMP) {
            if (half == 1) {
                const int nn = n0 + brow0 + 32 * j;
                const int kb = 2 * ts + (p >> 2);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int m = m0 + 64 * wm + 32 * i + mfma32_acc_row(v, g);
                    if (m < M && nn < N && kb < KB) dots[(int64_t(m) * N + nn) * KB + kb] = int(2.f * D[buf][v]);
                }
            }
        }
    };
    // the interleave of one product's MFMAs with the previous product's multiply-adds
    auto pattern = []() {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // VALU
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    };

    // One K-step on ring position R = s % 3.  On entry the step's min-term and block-0
    // operands are in registers (read right after the barrier that published the slot) and
    // the loads of step s + 1 are in flight.  The barrier that publishes step s + 1 comes
    // once block 0's products are issued: block 1's operands are in registers by then, so
    // the step's slot is no longer read and the barrier also frees it, and block 1's four
    // products hide the latency of the next step's first operand reads.
    auto step = [&](auto r_c, int s) {
        constexpr int R = decltype(r_c)::value, R1 = (R + 1) % 3, R2 = (R + 2) % 3;
        using RR2 = std::integral_constant<int, R2>;
        const int ts = sbeg + s;
        const int t2 = min(ts + 2, tlast);   // past the range: the last step again (never read)
        __builtin_amdgcn_sched_barrier(0);
        issue(RR2{}, std::integral_constant<int, 0>{}, t2);   // slot R2 was last read before the last barrier
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x8bf16_1k(mins.ma[i], mins.mb[j], acc[i][j], 0, 0, 0);
        mfma_s(cur0, 0, 0, S[0]);
        mfma_d(cur0, 0, 0, D[0]);
        load_ops(slot_at<R>(), 1, cur1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int p = 1; p < 8; ++p) {
            const Ops& o = p < 4 ? cur0 : cur1;
            const int i = (p >> 1) & 1, j = p & 1;
            mfma_s(o, i, j, S[p & 1]);
            fmas(p - 1, 0, ts);
            mfma_d(o, i, j, D[p & 1]);
            fmas(p - 1, 1, ts);
            pattern();
            if (p == 1) issue(RR2{}, std::integral_constant<int, 1>{}, t2);
            if (p == 2) issue(RR2{}, std::integral_constant<int, 2>{}, t2);
            if (p == 3) issue(RR2{}, std::integral_constant<int, 3>{}, t2);
            if (p == 4) {
                // Block 0's operands are dead: publish step s + 1 (past the last step:
                // harmless reads of a stale slot) and read its first operands while block
                // 1's products run.  Four loads of step s + 2 may still be in flight (the
                // block-dot export's stores count in vmcnt too: it waits for everything).
                if constexpr (DUMP) vmcnt_wait<0>();
                else vmcnt_wait<4>();
                lds_publish_barrier();
                load_min(slot_at<R1>(), mins);
                load_ops(slot_at<R1>(), 0, cur0);
            }
            if (p == 5) issue(RR2{}, std::integral_constant<int, 4>{}, t2);
            if (p == 6) issue(RR2{}, std::integral_constant<int, 5>{}, t2);
            if (p == 7) issue(RR2{}, std::integral_constant<int, 6>{}, t2);
            __builtin_amdgcn_sched_barrier(0);
        }
        fmas(7, 0, ts);
        fmas(7, 1, ts);
    };

    // prologue: steps 0 and 1 in flight, step 0 landed, published and its first operands read
    issue_all(std::integral_constant<int, 0>{}, sbeg);
    issue_all(std::integral_constant<int, 1>{}, min(sbeg + 1, tlast));
    vmcnt_wait<7>();
    lds_publish_barrier();
    load_min(g_slot0, mins);
    load_ops(g_slot0, 0, cur0);

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    for (int s = 0;;) {
        step(I0{}, s);
        if (++s >= nsteps) break;
        step(I1{}, s);
        if (++s >= nsteps) break;
        step(I2{}, s);
        if (++s >= nsteps) break;
    }
    vmcnt_wait<0>();   // no LDS-direct load of the ring may land after the workgroup ends

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
                    const int m = m0 + 64 * wm + 32 * i + mfma32_acc_row(v, g);
                    if (m < M && n < N) Y[int64_t(m) * N + n] = acc[i][j][v];
                }
            }
        return;
    }
    constexpr uint32_t kSlotBytes = BM * BN * sizeof(float);
    const __amdgpu_buffer_rsrc_t slots =
        raw_rsrc(partial + size_t(tile - full) * size_t(pieces) * (BM * BN), int64_t(pieces) * kSlotBytes);
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
                const int m = m0 + 64 * wm + 32 * i + mfma32_acc_row(v, g);
                if (m < M && n < N) Y[int64_t(m) * N + n] = y[j * 16 + v];
            }
        }
    }
}

template __global__ void mmq_f6_q4k_kernel<false>(const uint8_t* __restrict__, const uint8_t* __restrict__,
                                                  float* __restrict__, int32_t* __restrict__, float* __restrict__,
                                                  unsigned* __restrict__, int, int, int, int, int, int, int, int, int,
                                                  int);
template __global__ void mmq_f6_q4k_kernel<true>(const uint8_t* __restrict__, const uint8_t* __restrict__,
                                                 float* __restrict__, int32_t* __restrict__, float* __restrict__,
                                                 unsigned* __restrict__, int, int, int, int, int, int, int, int, int,
                                                 int);

}  // namespace

size_t mmq_f6_lds_bytes() { return 3 * sizeof(Slot) + 1024; }

MmqPlan mmq_f6_plan(int64_t M, int64_t N, int64_t K) {
    // As the int8 plan: tiles are dealt whole while they fill rounds of kTargetWorkgroups; the
    // tiles of a last round that is at most half full (or all tiles, when there are fewer
    // than half a round) are cut into K ranges of at least kMinStepsPerSplit steps, enough
    // for half a round: one workgroup per CU.  (Ranges for a full round, two per CU, were
    // slower on every shape timed: 7B ffn_up 104.4 against 95.0 us, 14B attn_q/o 147.3
    // against 136.7 us, with twice the partial tiles to sum.)  A function of the shape alone.
    MmqPlan p;
    p.bm = BM;
    p.steps = int((K + KS - 1) / KS);
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
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

size_t mmq_f6_scratch_bytes(int64_t M, int64_t N, int64_t K) {
    const MmqPlan p = mmq_f6_plan(M, N, K);
    return splitk_scratch_bytes(p.split_tiles, p.splits, int64_t(BM) * BN);
}

size_t mmq_f6_partial_bytes(int64_t M, int64_t N, int64_t K) {
    const MmqPlan p = mmq_f6_plan(M, N, K);
    return size_t(p.split_tiles) * size_t(p.splits) * size_t(BM) * BN * sizeof(float);
}

hipError_t launch_mmq_f6(const uint8_t* Wp, const uint8_t* Ap, float* Y, int32_t* dots, void* scratch,
                         unsigned* counters, int64_t M, int64_t N, int64_t K, hipStream_t s, const char** name) {
    *name = "mmq_f6<q4_K plane>";
    const MmqPlan plan = mmq_f6_plan(M, N, K);
    const int tiles_m = int((M + BM - 1) / BM);
    const int total = plan.full + plan.split_tiles * plan.splits;
    float* partial = static_cast<float*>(scratch);
    if (!counters && scratch) {   // the caller's scratch: counters, then the partial tiles
        counters = static_cast<unsigned*>(scratch);
        partial = reinterpret_cast<float*>(static_cast<uint8_t*>(scratch) + kSplitkCounterBytes);
    }
    const int Mp = int(f6_act_rows(M)), Np = int(f6_weight_rows(N));
    if (dots)
        hipLaunchKernelGGL(mmq_f6_q4k_kernel<true>, dim3(total), dim3(kThreads), 0, s, Wp, Ap, Y, dots, partial,
                           counters, int(M), int(N), int(K), Mp, Np, tiles_m, plan.full, plan.split_tiles,
                           plan.splits, plan.steps);
    else
        hipLaunchKernelGGL(mmq_f6_q4k_kernel<false>, dim3(total), dim3(kThreads), 0, s, Wp, Ap, Y, dots, partial,
                           counters, int(M), int(N), int(K), Mp, Np, tiles_m, plan.full, plan.split_tiles,
                           plan.splits, plan.steps);
    return hipGetLastError();
}

}  // namespace mq
