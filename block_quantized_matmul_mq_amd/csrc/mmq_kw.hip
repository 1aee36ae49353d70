// mq_gemm for Q4_K products with few output tiles (a small N, or a small M): the
// int8 "MMQ" prefill product ("minfer CUDA Backend Design", 4.4 Execution dispatch)
// with the K range of each output tile split over the waves of one workgroup.
//
//   Y[m][n] = sum_b dx[m][b] * ( dw[n][b] * D[m][n][b] - mw[n][b] * S[m][b] )
//
// (D: exact int32 dot of the weight and activation codes of 32-value block b; dx, S:
// the activation block's scale and code sum; dw = d * sc, mw = dmin * m: the Q4_K
// sub-block's scale and min.)
//
// Why.  Products with few 32 x 128 tiles (the 7B attn_k / attn_v at M = 512: 64 of them)
// have to cut K to fill 256 CUs, and summing K ranges across workgroups costs three
// serial trips to the device-coherent level (partials stored and acknowledged, the
// counter's atomic, the partials read back): about 4 us per launch.  Here a workgroup owns
// one 32 x 32 tile (four times as many tiles) and its waves take consecutive ranges of the
// K-steps; the ranges meet in LDS, so the only workgroup barrier is the one before the
// final sum.
//
// No LDS in the main loop.  The matrix unit's operand layout lets every lane fetch its own
// operands: for v_mfma_i32_32x32x32_i8, lane l supplies row l % 32 and values
// 16 (l / 32) .. +15 of a 32-value block, of both the activation tile (16 code bytes) and
// the weight tile, whose 16 bytes hold the codes of those values for two sub-blocks
// (low nibbles: sub-block 2c, high nibbles: 2c + 1).  Each lane therefore loads 16-byte
// pieces straight into registers, those of the next two K-steps in flight while one step
// is computed, and unpacks its own
// nibbles; it also decodes the scale and min of the sub-blocks it feeds to the scale
// products from the weight row's 16-byte header.  Per 128-value step a wave issues nine
// 16-byte loads per lane.
//
// The arithmetic per block pair is the int8 MMQ kernel's: block dots on
// v_mfma_i32_32x32x32_i8, the scale outer product dx (x) dw on v_mfma_f32_32x32x1_2b_f32,
// acc += float(D) * scale on the vector ALU, and the min term of the step's four blocks
// as one v_mfma_f32_32x32x16_bf16 over bf16 hi/lo splits, in the same order; the K ranges
// are summed in range order.  So a range split the same way gives the same bits.
#include <type_traits>

#include "mmq_common.h"
#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v32f __attribute__((ext_vector_type(32)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kTile = 32;     // output tile rows and columns
constexpr int kStep = 128;    // K values per step: four 32-value blocks, half a Q4_K super-block
constexpr int kWaves = 4;     // waves per workgroup, i.e. K ranges per tile (eight were slower)
constexpr int kXcds = 8;

// The waves' partial tiles, lane-major per accumulator element, for the final sum (the
// block-dot export sums nothing).
template <bool DUMP>
using Partials = float[DUMP ? 1 : kWaves][16][64];

// The operands one lane fetches for one K-step (row r = lane % 32, half h = lane / 32).
struct StepRegs {
    v4i a[4];   // activation codes of values 32 b + 16 h .. +15 of the step, blocks b = 0..3
    v4i q[2];   // weight code bytes 16 h .. +15 of the step's 64-value groups c = 0, 1
    v4i hd;     // the weight row's super-block header: d, dmin (f16), 12 bytes of packed scales
    v4i dx;     // activation block scales of the step's four blocks (f32 bits)
    v4i sum;    // activation code sums of the step's four blocks
};

struct Operands {
    __amdgpu_buffer_rsrc_t rc, rs, ru, rw;
    uint32_t va;    // lane offset into the activation codes: r K + 16 h
    uint32_t vs;    // into the scales and sums: 4 r KB
    uint32_t vw;    // into the weights: (weight row) row_bytes
    uint32_t vq;    // vw + 16 + 16 h: the lane's code bytes of a super-block's first group

    // in the order the step uses them
    __device__ void load(StepRegs& R, int s) const {
        const uint32_t k0 = uint32_t(s) * kStep;
        const uint32_t sb = uint32_t(s) >> 1, half = uint32_t(s) & 1;
        R.hd = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rw, vw, 144 * sb, 0));
        R.dx = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, vs, 16 * uint32_t(s), 0));
#pragma unroll
        for (int c = 0; c < 2; ++c)
            R.q[c] = __builtin_bit_cast(
                v4i, __builtin_amdgcn_raw_buffer_load_b128(rw, vq, 144 * sb + 64 * half + 32 * c, 0));
#pragma unroll
        for (int b = 0; b < 4; ++b)
            R.a[b] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rc, va, k0 + 32 * b, 0));
        R.sum = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(ru, vs, 16 * uint32_t(s), 0));
    }
};

// 6-bit scale and min of Q4_K sub-block j = 4 half + k (k = 0..3) from the header's
// packed bytes (s0, s1, s2 = dwords 1, 2, 3 of the header).  Both forms are formed and
// one is selected, so that a step is one basic block.
__device__ __forceinline__ void scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int half, int k, uint32_t& sc,
                                          uint32_t& mn) {
    const uint32_t sh = 8u * uint32_t(k);
    const uint32_t b_hi = (s2 >> sh) & 0xFFu;
    uint32_t sc_hi = (b_hi & 15u) | (((s0 >> (sh + 6)) & 3u) << 4);
    uint32_t mn_hi = (b_hi >> 4) | (((s1 >> (sh + 6)) & 3u) << 4);
    uint32_t sc_lo = (s0 >> sh) & 63u, mn_lo = (s1 >> sh) & 63u;
    // (opaque: otherwise the compiler turns the selects on the uniform `half` into branches)
    asm volatile("" : "+v"(sc_hi), "+v"(mn_hi), "+v"(sc_lo), "+v"(mn_lo));
    sc = half ? sc_hi : sc_lo;
    mn = half ? mn_hi : mn_lo;
}

template <bool DUMP>
struct Step {
    int h;
    int32_t* dots;
    int64_t dot_row0;   // for the export: (m0 + 8 (v / 4) + 4 h + v % 4) N + n0 + r, times KB, at v = 0
    int N, KB, m_rows, n_ok;

    // acc += the products of one K-step (step index s) of this lane's operands R
    __device__ void run(const StepRegs& R, int s, v16f& acc) const {
        const int half = s & 1;
        const uint32_t s0 = uint32_t(R.hd[1]), s1 = uint32_t(R.hd[2]), s2 = uint32_t(R.hd[3]);
        const float d = half_bits_to_float(uint32_t(R.hd[0]) & 0xFFFFu);
        const float dmin = half_bits_to_float(uint32_t(R.hd[0]) >> 16);
        // scale-outer-product operands: product p covers blocks 2p, 2p + 1, lane half h feeds
        // block 2p + h
        float sdx[2], sdw[2];
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            sdx[p] = __builtin_bit_cast(float, h ? R.dx[2 * p + 1] : R.dx[2 * p]);
            uint32_t sc, mn;
            scale_min(s0, s1, s2, half, 2 * p + h, sc, mn);
            sdw[p] = d * float(sc);
        }
        // weight operands of the step's blocks: group c's low nibbles are block 2c, its high
        // nibbles block 2c + 1
        v4i B[4];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                B[2 * c][e] = R.q[c][e] & 0x0F0F0F0F;
                B[2 * c + 1][e] = (int(uint32_t(R.q[c][e]) >> 4)) & 0x0F0F0F0F;
            }
        const v32f z32 = {};
        const v16i zi = {};
        v32f S[2];
        v16i D0, D1;
        S[0] = __builtin_amdgcn_mfma_f32_32x32x1f32(sdx[0], sdw[0], z32, 0, 0, 0);
        D0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(R.a[0], B[0], zi, 0, 0, 0);
        D1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(R.a[1], B[1], zi, 0, 0, 0);
        S[1] = __builtin_amdgcn_mfma_f32_32x32x1f32(sdx[1], sdw[1], z32, 0, 0, 0);
        auto consume = [&](const v16i& D, const v32f& Sp, int hh, int b) {
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[v] = fmaf(float(D[v]), Sp[16 * hh + v], acc[v]);
            asm volatile("" : "+v"(acc));
            if constexpr (DUMP) {
                const int kb = 4 * s + b;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int mr = 8 * (v >> 2) + 4 * h + (v & 3);
                    if (mr < m_rows && n_ok)
                        dots[(dot_row0 + int64_t(8 * (v >> 2) + (v & 3)) * N) * KB + kb] = D[v];
                }
            }
        };
        __builtin_amdgcn_sched_barrier(0);
        consume(D0, S[0], 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        D0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(R.a[2], B[2], zi, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        consume(D1, S[0], 1, 1);
        __builtin_amdgcn_sched_barrier(0);
        D1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(R.a[3], B[3], zi, 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        consume(D0, S[1], 0, 2);
        __builtin_amdgcn_sched_barrier(0);
        consume(D1, S[1], 1, 3);
        __builtin_amdgcn_sched_barrier(0);
        // min term of blocks 2h, 2h + 1 (this lane's half of the bf16 operands):
        // acc += sum_b tx[m][b] mw[n][b], tx = dx S and mw = -dmin m as bf16 hi / lo
        uint32_t t[2], w[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int b = 2 * h + i;
            const float dxb = __builtin_bit_cast(float, h ? R.dx[2 + i] : R.dx[i]);
            const int32_t sb = h ? R.sum[2 + i] : R.sum[i];
            t[i] = bf16_hilo_bits(dxb * float(sb));
            uint32_t sc, mn;
            scale_min(s0, s1, s2, half, b, sc, mn);
            w[i] = bf16_hilo_bits(-(dmin * float(mn)));
        }
        const v4i am = {int((t[0] & 0xFFFFu) | (t[0] << 16)), int(t[0] >> 16), int((t[1] & 0xFFFFu) | (t[1] << 16)),
                        int(t[1] >> 16)};
        const v4i bm = {int(w[0]), int(w[0] & 0xFFFFu), int(w[1]), int(w[1] & 0xFFFFu)};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, am), __builtin_bit_cast(v8bf, bm), acc,
                                                      0, 0, 0);
    }
};

// One workgroup of kWaves waves per 32 x 32 output tile; wave w takes K-steps
// [w S / kWaves, (w + 1) S / kWaves) of the S = K / 128 steps.  Two workgroups fit on a
// CU (at most 256 registers a lane); the block-dot export keeps more registers instead.
template <bool DUMP>
__global__ __launch_bounds__(64 * kWaves, DUMP ? 1 : 2) void mmq_kw_q4k_kernel(const uint8_t* __restrict__ W,
                                                                           const int8_t* __restrict__ codes,
                                                                           const float* __restrict__ xscale,
                                                                           const int32_t* __restrict__ xsum,
                                                                           float* __restrict__ Y,
                                                                           int32_t* __restrict__ dots, int M, int N,
                                                                           int K, int64_t row_bytes, int tiles_n,
                                                                           int tiles) {
    __shared__ Partials<DUMP> red;
    // workgroups dealt to one XCD take consecutive tiles: the tiles of one row of tiles
    // share its activation rows
    const int id = blockIdx.x;
    const int tile = tiles % kXcds == 0 ? (id % kXcds) * (tiles / kXcds) + id / kXcds : id;
    const int m0 = (tile / tiles_n) * kTile, n0 = (tile % tiles_n) * kTile;
    // the wave index as a scalar: the K-step offsets go into the loads' scalar operand
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int r = lane & 31, h = lane >> 5;
    const int KB = K >> 5;
    const int steps = K / kStep;
    const int s0 = int(int64_t(wave) * steps / kWaves), s1 = int(int64_t(wave + 1) * steps / kWaves);

    const int rows = min(kTile, M - m0), cols = min(kTile, N - n0);
    Operands op;
    op.rc = raw_rsrc(codes + int64_t(m0) * K, int64_t(rows) * K);
    op.rs = raw_rsrc(xscale + int64_t(m0) * KB, int64_t(rows) * KB * 4);
    op.ru = raw_rsrc(xsum + int64_t(m0) * KB, int64_t(rows) * KB * 4);
    op.rw = raw_rsrc(W + int64_t(n0) * row_bytes, int64_t(cols) * row_bytes);
    // rows past M read zeros (out of the buffer's range); rows past N re-read the last row
    op.va = uint32_t(r * K + 16 * h);
    op.vs = uint32_t(4 * r * KB);
    op.vw = uint32_t(min(r, cols - 1) * row_bytes);
    op.vq = op.vw + 16 + 16 * h;

    Step<DUMP> st;
    st.h = h;
    st.dots = dots;
    st.N = N;
    st.KB = KB;
    st.m_rows = rows;
    st.n_ok = r < cols;
    st.dot_row0 = int64_t(m0 + 4 * h) * N + n0 + r;

    v16f acc;
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[v] = 0.f;

    if (s0 < s1) {
        // three register sets: the step being computed and the next two in flight; loads
        // past the range re-read its last step (same count every step, no branches)
        const int last = s1 - 1;
        StepRegs A, B, C;
        // (the scheduling barriers keep the sets' loads in issue order, so that the waits
        // before each step count exactly the two later sets)
        op.load(A, s0);
        __builtin_amdgcn_sched_barrier(0);
        op.load(B, min(s0 + 1, last));
        // whole groups of three steps, then the last one or two
        int s = s0;
        for (; s + 3 <= s1; s += 3) {
            __builtin_amdgcn_sched_barrier(0);
            op.load(C, min(s + 2, last));
            __builtin_amdgcn_sched_barrier(0);
            st.run(A, s, acc);
            __builtin_amdgcn_sched_barrier(0);
            op.load(A, min(s + 3, last));
            __builtin_amdgcn_sched_barrier(0);
            st.run(B, s + 1, acc);
            __builtin_amdgcn_sched_barrier(0);
            op.load(B, min(s + 4, last));
            __builtin_amdgcn_sched_barrier(0);
            st.run(C, s + 2, acc);
        }
        if (s < s1) st.run(A, s, acc);
        if (s + 1 < s1) st.run(B, s + 1, acc);
    }
    if constexpr (DUMP) return;

    // the waves' partial tiles, summed in wave (K) order
#pragma unroll
    for (int v = 0; v < 16; ++v) red[wave][v][lane] = acc[v];
    __syncthreads();
#pragma unroll
    for (int e0 = 0; e0 < 16 * 64; e0 += 64 * kWaves) {
        const int e = e0 + int(threadIdx.x);
        const int v = e >> 6, l = e & 63;
        float y = red[0][v][l];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) y += red[w][v][l];
        const int mr = mfma32_acc_row(v, l >> 5), nc = l & 31;
        if (mr < rows && nc < cols) Y[int64_t(m0 + mr) * N + n0 + nc] = y;
    }
}

// Explicit instantiations (the launch stubs are otherwise not emitted when the kernels are
// only named inside the launcher).
#define MQ_KW_INSTANCE(DUMP)                                                                                  \
    template __global__ void mmq_kw_q4k_kernel<DUMP>(const uint8_t* __restrict__, const int8_t* __restrict__,  \
                                                     const float* __restrict__, const int32_t* __restrict__,   \
                                                     float* __restrict__, int32_t* __restrict__, int, int, int, \
                                                     int64_t, int, int);
MQ_KW_INSTANCE(false)
MQ_KW_INSTANCE(true)
#undef MQ_KW_INSTANCE

}  // namespace

size_t mmq_kw_lds_bytes() { return sizeof(Partials<false>); }

bool mmq_kw_applies(int type, BlockLayout lay, int64_t M, int64_t N, int64_t K) {
    if (type != kQ4_K || lay.stride != 144 || lay.off != 0 || M <= kGemvQ8MaxRows || K % kStep != 0) return false;
    // Where the int8 kernel takes 32 x 128 tiles that do not fill half of its 512-workgroup
    // round (it then cuts them into K ranges summed across workgroups, or leaves CUs idle).
    // A step costs about 0.9 us in either kernel (one wave per SIMD), and the cross-workgroup
    // sum about 4.3 us, i.e. five steps: this kernel is taken unless its waves would run more
    // than five steps beyond the int8 kernel's longest range.  (Timed, M x N x K:
    // 512 x 512 x 3584 9.9 against 14.7 us, 512 x 1024 x 3584 16.5 against 19.4,
    // 20 x 3000 x 3584 8.4 against 12.0, 200 x 2560 x 2560 (140 tiles, none cut) 16.1
    // against 25.1.  With 448 tiles, none cut (512 x 3584 x 3584), it took 59 against 41 us,
    // so it is not used there.)
    const MmqPlan p = mmq_plan(type, M, N, K);
    if (p.bm != 32 || int64_t(p.full) + p.split_tiles > 256) return false;
    const int64_t tiles = ((M + kTile - 1) / kTile) * ((N + kTile - 1) / kTile);
    const int64_t rounds = (tiles + 511) / 512;   // two resident workgroups per CU
    const int64_t kw_steps = (p.steps + 3) / 4 * rounds;
    const int64_t range_steps = (p.steps + p.splits - 1) / p.splits;
    return kw_steps <= range_steps + 5;
}

hipError_t launch_mmq_kw(const uint8_t* W, const int8_t* codes, const float* xs, const int32_t* xsum, float* Y,
                         int32_t* dots, int64_t M, int64_t N, int64_t K, hipStream_t s, const char** name) {
    const int tiles_m = int((M + kTile - 1) / kTile), tiles_n = int((N + kTile - 1) / kTile);
    const int tiles = tiles_m * tiles_n;
    const int64_t row_bytes = (K / 256) * 144;
    *name = "mmq_kw<q4_K>";
    if (dots)
        hipLaunchKernelGGL((mmq_kw_q4k_kernel<true>), dim3(tiles), dim3(64 * kWaves), 0, s, W, codes, xs, xsum, Y,
                           dots, int(M), int(N), int(K), row_bytes, tiles_n, tiles);
    else
        hipLaunchKernelGGL((mmq_kw_q4k_kernel<false>), dim3(tiles), dim3(64 * kWaves), 0, s, W, codes, xs, xsum, Y,
                           dots, int(M), int(N), int(K), row_bytes, tiles_n, tiles);
    return hipGetLastError();
}

}  // namespace mq
