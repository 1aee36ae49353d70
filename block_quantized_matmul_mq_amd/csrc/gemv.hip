// mq_gemv kernels: y = deq(W) x for one f32 activation row (the decode
// product of "minfer CUDA Backend Design", 4.4 Execution dispatch).
//
// Work split.  One 1024-thread workgroup per compute unit owns a contiguous
// range of output rows (the grid is balanced to within one row per CU).  Each
// row is cut into "units" (Q4_K and Q6_K: 64 values; Q8_0: one 32-value block)
// and the rows x units of the range are dealt to the 1024 lanes round-robin,
// so consecutive lanes read consecutive weight bytes and every lane gets the
// same amount of work whatever the row length.  A lane writes one f32 partial
// per unit to LDS; the partials of a row are then summed by a fixed group of
// lanes in a fixed order, so the result is deterministic.
//
// Activation.  The workgroup first stages x in LDS in an exact integer form:
// per 32-value block b, x = 2^e_b * v with v = rint(x * 2^-e_b) an integer of at
// most 21 bits (e_b puts the block maximum in [2^20, 2^21)), so the staged
// value differs from x by at most 2^-21 of the block maximum (f32-grade).  v is
// kept as three signed bytes (v = 65536 d2 + 256 d1 + d0) in three byte planes,
// which lets the weight codes meet x in v_dot4_i32_i8: three dot4 per four
// codes, exact int32 sums, one conversion to f32 per run of codes that shares a
// scale.  Q4_K, Q5_K and the 32-value types also need the f32 sum of x over each
// 32-block (their min term or code offset); Q6_K the sum over each 16-value run
// (code offset 32).
#include <cstdio>
#include <cstdlib>

#include "mq_device.h"
#include "mq_internal.h"
#include "weight_units.h"

namespace mq {

namespace {

constexpr int kFracBits = 21;

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4(int(a), int(b), c, false);
}

// exact: sum_i code_i * v_i for the three digit planes
__device__ __forceinline__ float combine3(int a2, int a1, int a0) {
    return fmaf(float(a2), 65536.0f, fmaf(float(a1), 256.0f, float(a0)));
}

// Staged x (LDS).  Each plane holds one signed digit per value, grouped in
// 16-value chunks laid out unit-major: chunk k of unit u sits at byte
// (k * S + u) * 16 with S = units + 1.  Lanes own consecutive units, so one
// ds_read_b128 per lane touches consecutive 16-byte chunks: no bank conflicts.
struct Stage {
    const uint8_t* p0;
    const uint8_t* p1;
    const uint8_t* p2;
    int S;               // chunk-row stride, in chunks
    const int* ex;       // block exponent: per 32-block (Q4_K, Q8_0), per (unit, t) (Q6_K)
    const float* sums;   // f32 sum of x: per 32-block (Q4_K), per (unit, t) 16-run (Q6_K)

    __device__ void chunk(int k, int u, uint4& a, uint4& b, uint4& c) const {
        const int off = (k * S + u) * 16;
        a = *reinterpret_cast<const uint4*>(p0 + off);
        b = *reinterpret_cast<const uint4*>(p1 + off);
        c = *reinterpret_cast<const uint4*>(p2 + off);
    }
};

// Dot of 16 codes (4 dwords, one byte each) with one staged chunk, per plane.
__device__ __forceinline__ void dot16(const uint32_t* c, const uint4& a, const uint4& b, const uint4& e,
                                      int& s0, int& s1, int& s2) {
    s0 = sdot4(c[0], a.x, s0); s0 = sdot4(c[1], a.y, s0); s0 = sdot4(c[2], a.z, s0); s0 = sdot4(c[3], a.w, s0);
    s1 = sdot4(c[0], b.x, s1); s1 = sdot4(c[1], b.y, s1); s1 = sdot4(c[2], b.z, s1); s1 = sdot4(c[3], b.w, s1);
    s2 = sdot4(c[0], e.x, s2); s2 = sdot4(c[1], e.y, s2); s2 = sdot4(c[2], e.z, s2); s2 = sdot4(c[3], e.w, s2);
}

// ---------------------------------------------------------------- Q4_K
// Staged chunks 0,1 hold values 64u..64u+31 (the low nibbles), chunks 2,3 values
// 64u+32..64u+63.
struct UnitQ4K : RawQ4K {
    static constexpr int kChunks = 4;

    // exact sum of code * v over a 32-value run: int32 (|s2| <= 32 * 15 * 32)
    __device__ static int run_dot(const uint32_t (&c)[8], const Stage& st, int k0, int uu) {
        int s0 = 0, s1 = 0, s2 = 0;
        uint4 a, b, e;
        st.chunk(k0, uu, a, b, e);
        dot16(c, a, b, e, s0, s1, s2);
        st.chunk(k0 + 1, uu, a, b, e);
        dot16(c + 4, a, b, e, s0, s1, s2);
        return (s2 << 16) + (s1 << 8) + s0;
    }

    __device__ float dot(const Stage& st, int uu, int u) const {
        uint32_t lo[8], hi[8];
        codes(lo, hi);
        const int ilo = run_dot(lo, st, 0, uu);
        const int ihi = run_dot(hi, st, 2, uu);
        uint32_t scp, mnp;
        scale_min(u & 3, scp, mnp);
        const int2 e2 = *reinterpret_cast<const int2*>(st.ex + 2 * uu);
        const float2 s2 = *reinterpret_cast<const float2*>(st.sums + 2 * uu);
        const float codes_term = ldexpf(ubyte_f<0>(scp) * float(ilo), e2.x) + ldexpf(ubyte_f<1>(scp) * float(ihi), e2.y);
        const float mins = fmaf(ubyte_f<0>(mnp), s2.x, ubyte_f<1>(mnp) * s2.y);
        return fmaf(d(), codes_term, -dmin() * mins);
    }
};

// ---------------------------------------------------------------- Q5_K
// As Q4_K, with 5-bit codes (|sum code * v| <= 32 * 31 * 2^21 < 2^31 over a run).
struct UnitQ5K : RawQ5K {
    static constexpr int kChunks = 4;

    __device__ float dot(const Stage& st, int uu, int u) const {
        uint32_t lo[8], hi[8];
        codes(u, lo, hi);
        const int ilo = UnitQ4K::run_dot(lo, st, 0, uu);
        const int ihi = UnitQ4K::run_dot(hi, st, 2, uu);
        uint32_t scp, mnp;
        scale_min(u & 3, scp, mnp);
        const int2 e2 = *reinterpret_cast<const int2*>(st.ex + 2 * uu);
        const float2 s2 = *reinterpret_cast<const float2*>(st.sums + 2 * uu);
        const float codes_term = ldexpf(ubyte_f<0>(scp) * float(ilo), e2.x) + ldexpf(ubyte_f<1>(scp) * float(ihi), e2.y);
        const float mins = fmaf(ubyte_f<0>(mnp), s2.x, ubyte_f<1>(mnp) * s2.y);
        return fmaf(d(), codes_term, -dmin() * mins);
    }
};

// ---------------------------------------------------------------- Q4_0 / Q4_1 / Q5_0 / Q5_1
// Staged chunks 0,1 hold the block's 32 values.  sum((code - offset) * x) =
// 2^e * sum(code * v) - offset * sum(x); the min of Q4_1 / Q5_1 adds m * sum(x).
template <int QT>
struct UnitLegacy : RawLegacy<QT> {
    static constexpr int kChunks = 2;

    __device__ float dot(const Stage& st, int uu, int) const {
        uint32_t c[8];
        this->codes(c);
        int s0 = 0, s1 = 0, s2 = 0;
        uint4 a, b, e;
        st.chunk(0, uu, a, b, e);
        dot16(c, a, b, e, s0, s1, s2);
        st.chunk(1, uu, a, b, e);
        dot16(c + 4, a, b, e, s0, s1, s2);
        const float cv = ldexpf(combine3(s2, s1, s0), st.ex[uu]);
        const float sx = st.sums[uu];
        if constexpr (Legacy<QT>::kMin) return fmaf(this->d(), cv, this->m() * sx);
        return this->d() * fmaf(-float(Legacy<QT>::kOffset), sx, cv);
    }
};

// ---------------------------------------------------------------- Q6_K
// Staged chunk t of the unit holds exactly the 16 values of run t.
struct UnitQ6K : RawQ6K {
    static constexpr int kChunks = 4;

    __device__ float dot(const Stage& st, int uu, int u) const {
        uint32_t A[4], B[4], H[4], s0, s1;
        realign(A, B, H, s0, s1);
        const int4 e4 = *reinterpret_cast<const int4*>(st.ex + 4 * uu);
        const float4 m4 = *reinterpret_cast<const float4*>(st.sums + 4 * uu);
        const int ev[4] = {e4.x, e4.y, e4.z, e4.w};
        const float sv[4] = {m4.x, m4.y, m4.z, m4.w};
        float acc = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint32_t code[4];
            run_codes(t, A, B, H, code);
            uint4 xa, xb, xc;
            st.chunk(t, uu, xa, xb, xc);
            int d0 = 0, d1 = 0, d2 = 0;
            dot16(code, xa, xb, xc, d0, d1, d2);
            // sum((c - 32) * x) = 2^e * sum(c * v) - 32 * sum(x)
            const float cv = ldexpf(combine3(d2, d1, d0), ev[t]);
            acc = fmaf(subscale(t, u, s0, s1), fmaf(-32.0f, sv[t], cv), acc);
        }
        return d() * acc;
    }
};

// ---------------------------------------------------------------- Q8_0
// Staged chunks 0,1 hold the block's 32 values.
struct UnitQ80 : RawQ80 {
    static constexpr int kChunks = 2;

    __device__ float dot(const Stage& st, int uu, int) const {
        uint32_t c[8];
        codes(c);
        int s0 = 0, s1 = 0, s2 = 0;
        uint4 a, b, e;
        st.chunk(0, uu, a, b, e);
        dot16(c, a, b, e, s0, s1, s2);
        st.chunk(1, uu, a, b, e);
        dot16(c + 4, a, b, e, s0, s1, s2);
        return d() * ldexpf(combine3(s2, s1, s0), st.ex[uu]);
    }
};

template <int QT> struct UnitOf;
template <> struct UnitOf<kQ4_K> { using T = UnitQ4K; };
template <> struct UnitOf<kQ6_K> { using T = UnitQ6K; };
template <> struct UnitOf<kQ8_0> { using T = UnitQ80; };
template <> struct UnitOf<kQ5_K> { using T = UnitQ5K; };
template <> struct UnitOf<kQ4_0> { using T = UnitLegacy<kQ4_0>; };
template <> struct UnitOf<kQ4_1> { using T = UnitLegacy<kQ4_1>; };
template <> struct UnitOf<kQ5_0> { using T = UnitLegacy<kQ5_0>; };
template <> struct UnitOf<kQ5_1> { using T = UnitLegacy<kQ5_1>; };

__device__ __forceinline__ float group_sum(float v, int width) {
    for (int off = width >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Byte k of four dwords -> one dword (a 4 x 4 byte transpose, three planes).
__device__ __forceinline__ void transpose_digits(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3,
                                                 uint32_t& p0, uint32_t& p1, uint32_t& p2) {
    const uint32_t t01 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);   // r0.b0 r1.b0 r0.b1 r1.b1
    const uint32_t t23 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
    p0 = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
    p1 = __builtin_amdgcn_perm(t23, t01, 0x07060302u);
    const uint32_t u01 = __builtin_amdgcn_perm(r1, r0, 0x00000602u);   // r0.b2 r1.b2
    const uint32_t u23 = __builtin_amdgcn_perm(r3, r2, 0x00000602u);
    p2 = __builtin_amdgcn_perm(u23, u01, 0x05040100u);
}

// Signed digits of v = rint(x * 2^k) (|v| < 2^21) in bytes 0..2:
// (v + 0x808080) has unsigned bytes b_i = d_i + 128, and b_i ^ 0x80 is d_i as int8.
__device__ __forceinline__ uint32_t digits(float x, int k) {
    const float f = ldexpf(x, k) + 12582912.0f;   // 1.5 * 2^23: the low mantissa bits are rint(x*2^k)
    return (__float_as_uint(f) - 0x4ABF7F80u) ^ 0x00808080u;
}

// LDS layout (dynamic): three digit planes of plane_bytes(K) | block exponents
// int | sums f32 | partials f32 [tile_units]  (see lds_layout below)
template <int QT, int kThreads, int kSlots>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const uint8_t* __restrict__ W,
                                                        const float* __restrict__ x,
                                                        float* __restrict__ y, int N, int K,
                                                        int64_t row_bytes, int tile_units, int blk_stride,
                                                        int blk_off) {
    using Unit = typename UnitOf<QT>::T;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int U = K / Unit::kValues;
    const int S = U + 1;
    const int plane = Unit::kChunks * S * 16;
    uint8_t* p0 = smem;
    uint8_t* p1 = p0 + plane;
    uint8_t* p2 = p1 + plane;
    int* ex = reinterpret_cast<int*>(p2 + plane);
    const int nex = (QT == kQ6_K) ? 4 * U : (K >> 5);
    float* sums = reinterpret_cast<float*>(ex + nex);
    const int nsum = (QT == kQ6_K) ? 4 * U : (QT == kQ8_0 ? 0 : (K >> 5));
    float* part = sums + nsum;

    const int tid = threadIdx.x;
    const int r_begin = int((int64_t(blockIdx.x) * N) / gridDim.x);
    const int r_end = int((int64_t(blockIdx.x + 1) * N) / gridDim.x);
    const int rows_per_tile = max(1, tile_units / U);

    // A lane handles flat unit indices f = tid, tid + kThreads, ... of a tile.
    // The loads run kSlots units ahead of the computes through a ring of unit
    // buffers; two cursors (next load, next compute) step by kThreads units
    // without multiplies or divisions.
    const int dq = kThreads / U, dr = kThreads - dq * U;
    const int64_t dq_bytes = int64_t(dq) * row_bytes;
    struct Cursor {
        int f, u;
        const uint8_t* row;
    };
    auto start = [&](Cursor& c, const uint8_t* tile) {
        c.f = tid;
        const int r = tid / U;
        c.u = tid - r * U;
        c.row = tile + int64_t(r) * row_bytes;
    };
    auto advance = [&](Cursor& c) {
        c.f += kThreads;
        c.u += dr;
        c.row += dq_bytes;
        if (c.u >= U) {
            c.u -= U;
            c.row += row_bytes;
        }
    };

    // A tile takes `iters` rounds of kThreads units (the last round partly dead).  The
    // steady part of the loop issues every slot load unconditionally (a dead lane of the
    // last round re-reads the tile's first unit, valid and cached), so the number of
    // loads in flight is static and the compiler waits for exactly the slot it needs
    // (loads complete in issue order); only the drain at the end of a tile, which issues
    // no loads past the tile, waits for all.
    Unit buf[kSlots];
    Cursor ld, cp;
    int t0 = r_begin;
    const uint8_t* tile = W + int64_t(t0) * row_bytes;
    int units = 0, iters = 0;
    auto load_next = [&](int j) {
        const bool live = ld.f < units;
        buf[j].load(live ? ld.row : tile, live ? ld.u : 0, blk_stride, blk_off);
        advance(ld);
    };
    auto prime = [&](int tfirst) {
        units = min(rows_per_tile, r_end - tfirst) * U;
        iters = (units + kThreads - 1) / kThreads;
        tile = W + int64_t(tfirst) * row_bytes;
        start(ld, tile);
        start(cp, tile);
#pragma unroll
        for (int j = 0; j < kSlots; ++j) load_next(j);
    };
    // x first: loads complete in issue order, so x must be requested before the
    // weight prefetch or staging it would wait for all of that prefetch.
    constexpr int kEarly = 32768 / 4 / kThreads;   // covers every K the LDS can stage
    const int nquads = K >> 2;
    float4 xe[kEarly];
#pragma unroll
    for (int e = 0; e < kEarly; ++e) {
        const int i = tid + e * kThreads;
        if (i < nquads) xe[e] = reinterpret_cast<const float4*>(x)[i];
    }
    // Then the first tile's weight loads.
    prime(t0);

    // Stage x: 8 lanes per 32-block, 4 values (one float4) per lane.
    auto stage = [&](int i, const float4 v) {
        float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        a = lanes8_max(a);   // (DPP within groups of 8 lanes, all active or all idle)
        // amax = m * 2^E, m in [0.5, 1): scale by 2^(21 - E) puts the block in [2^20, 2^21)
        const int k = kFracBits - __builtin_amdgcn_frexp_expf(a);
        uint32_t d0, d1, d2;
        transpose_digits(digits(v.x, k), digits(v.y, k), digits(v.z, k), digits(v.w, k), d0, d1, d2);
        // unit and chunk of values 4i .. 4i+3
        const int val = 4 * i;
        int uu, kc;
        if constexpr (QT == kQ6_K) {
            uu = ((val >> 8) << 2) | (((val >> 7) & 1) << 1) | ((val >> 4) & 1);
            kc = (val >> 5) & 3;
        } else if constexpr (QT == kQ4_K || QT == kQ5_K) {
            uu = val >> 6;
            kc = (val >> 4) & 3;
        } else {
            uu = val >> 5;
            kc = (val >> 4) & 1;
        }
        const int off = (kc * S + uu) * 16 + 4 * (i & 3);
        *reinterpret_cast<uint32_t*>(p0 + off) = d0;
        *reinterpret_cast<uint32_t*>(p1 + off) = d1;
        *reinterpret_cast<uint32_t*>(p2 + off) = d2;
        float sm = (v.x + v.y) + (v.z + v.w);
        sm = lanes8_sum<2>(sm);
        if constexpr (QT == kQ6_K) {
            if ((i & 3) == 0) {            // one 16-run = chunk kc of unit uu
                sums[4 * uu + kc] = sm;
                ex[4 * uu + kc] = -k;
            }
        } else {
            if constexpr (QT != kQ8_0) {
                sm += dpp8_partner<2>(sm);   // the other four lanes of the 32-block
                if ((i & 7) == 0) sums[i >> 3] = sm;
            }
            if ((i & 7) == 0) ex[i >> 3] = -k;
        }
    };
    // (groups of 8 lanes are either all below nquads or all above: K % 32 == 0)
#pragma unroll
    for (int e = 0; e < kEarly; ++e) {
        const int i = tid + e * kThreads;
        if (i < nquads) stage(i, xe[e]);
    }
    for (int i = tid + kEarly * kThreads; i < nquads; i += kThreads)
        stage(i, reinterpret_cast<const float4*>(x)[i]);
    __syncthreads();

    const Stage st{p0, p1, p2, S, ex, sums};

    for (; t0 < r_end; t0 += rows_per_tile) {
        const int rows = min(rows_per_tile, r_end - t0);

        int it0 = 0;
        for (; it0 + 2 * kSlots <= iters; it0 += kSlots) {
#pragma unroll
            for (int j = 0; j < kSlots; ++j) {
                if (cp.f < units) part[cp.f] = buf[j].dot(st, cp.u, cp.u);
                advance(cp);
                load_next(j);   // round it0 + j + kSlots < iters: always a round of this tile
            }
        }
        // drain: the last rounds, loading only rounds that exist (the conditions are uniform)
#pragma unroll
        for (int j = 0; j < 2 * kSlots; ++j) {
            if (it0 + j < iters) {
                if (cp.f < units) part[cp.f] = buf[j % kSlots].dot(st, cp.u, cp.u);
                advance(cp);
                if (it0 + j + kSlots < iters) load_next(j % kSlots);
            }
        }
        // Issue the next tile's first loads before summing this one.
        const int t1 = t0 + rows_per_tile;
        if (t1 < r_end) prime(t1);
        __syncthreads();

        // Row sums: `width` lanes per row, each summing a strided slice, then a shuffle tree.
        int width = 64;
        while (width > 1 && (kThreads / width) < rows) width >>= 1;
        const int groups = kThreads / width;
        const int lane_in = tid & (width - 1);
        const int padded = rows + (groups - rows % groups) % groups;
        for (int r = tid / width; r < padded; r += groups) {
            float s = 0.f;
            if (r < rows) {
                const float* pr = part + r * U;
                for (int j = lane_in; j < U; j += width) s += pr[j];
            }
            s = group_sum(s, width);
            if (r < rows && lane_in == 0) y[t0 + r] = s;
        }
        __syncthreads();
    }
}

// Threads per workgroup and ring depth of the vector kernel (every type).
constexpr int kGemvThreads = 1024;
constexpr int kGemvSlots = 2;

template <int QT>
const void* kernel_ptr() {
    return reinterpret_cast<const void*>(gemv_kernel<QT, kGemvThreads, kGemvSlots>);
}

const void* kernel_for(int type) {
    switch (type) {
        case kQ4_K: return kernel_ptr<kQ4_K>();
        case kQ5_K: return kernel_ptr<kQ5_K>();
        case kQ6_K: return kernel_ptr<kQ6_K>();
        case kQ8_0: return kernel_ptr<kQ8_0>();
        case kQ4_0: return kernel_ptr<kQ4_0>();
        case kQ4_1: return kernel_ptr<kQ4_1>();
        case kQ5_0: return kernel_ptr<kQ5_0>();
        case kQ5_1: return kernel_ptr<kQ5_1>();
        default: return nullptr;
    }
}

}  // namespace

size_t fixed_lds_bytes(int type, int64_t K) {
    const int64_t vals = unit_values(type);
    const int64_t chunks = vals / 16;
    const int64_t U = K / vals;
    size_t b = 3 * size_t(chunks * (U + 1) * 16);            // digit planes
    b += size_t(type == kQ6_K ? 4 * U : K / 32) * 4;         // exponents
    if (type == kQ6_K) b += size_t(4 * U) * 4;               // sums per (unit, 16-run)
    else if (type != kQ8_0) b += size_t(K / 32) * 4;         // sums per 32-block
    return b;
}

// Largest tile (in units) that fits next to the staged x; 0 if not even one row fits.
int gemv_tile_units(int type, int64_t K, size_t lds_limit) {
    const size_t fixed = fixed_lds_bytes(type, K);
    const int vals = unit_values(type);
    const int64_t U = K / vals;
    if (lds_limit <= fixed) return 0;
    int64_t units = int64_t((lds_limit - fixed) / 4);
    if (units > 65536) units = 65536;
    if (units < U) return 0;
    return int(units);
}

hipError_t gemv_set_attributes(size_t lds_limit) {
    for (int type : {kQ4_K, kQ5_K, kQ6_K, kQ8_0, kQ4_0, kQ4_1, kQ5_0, kQ5_1}) {
        hipError_t e = hipFuncSetAttribute(kernel_for(type), hipFuncAttributeMaxDynamicSharedMemorySize,
                                           int(lds_limit));
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_gemv(int type, BlockLayout layout, const uint8_t* W, const float* x, float* y, int64_t N,
                       int64_t K, hipStream_t s, const char** name) {
    const DeviceInfo* info = device_info();
    if (!info) return hipErrorInvalidDevice;
    if (type == kQ4_K && gemv_mfma_applies(type, N, K, info->cu_count))
        return launch_gemv_mfma(W, x, y, N, K, info->cu_count, s, name);
    if (gemv_tiled_applies(type, layout, W, N, K, info->cu_count))
        return launch_gemv_tiled(type, W, x, y, N, K, info->cu_count, s, name);
    if (gemv_wide_applies(type, layout, W, N, K, info->cu_count))
        return launch_gemv_wide(type, W, x, y, N, K, info->cu_count, s, name);
    int tile = gemv_tile_units(type, K, info->lds_per_block);
    if (tile <= 0) return hipErrorInvalidValue;
    const int vals = unit_values(type);
    const int U = int(K / vals);
    // Rows of one workgroup; shrink the tile so a workgroup's rows split into equal tiles.
    const int grid = int(N < info->cu_count ? N : info->cu_count);
    const int64_t rows_wg = (N + grid - 1) / grid;
    const int64_t max_rows = tile / U;
    const int64_t ntiles = (rows_wg + max_rows - 1) / max_rows;
    const int64_t rows_tile = (rows_wg + ntiles - 1) / ntiles;
    tile = int(rows_tile * U);
    const size_t shmem = fixed_lds_bytes(type, K) + size_t(tile) * 4;
    const void* kern = kernel_for(type);
    const bool repacked = layout.off != 0 || (type == kQ6_K && layout.stride != 210);
    switch (type) {
        case kQ8_0: *name = repacked ? "gemv<q8_0 repacked>" : "gemv<q8_0>"; break;
        case kQ4_K: *name = "gemv<q4_K>"; break;
        case kQ5_K: *name = "gemv<q5_K>"; break;
        case kQ6_K: *name = repacked ? "gemv<q6_K repacked>" : "gemv<q6_K>"; break;
        case kQ4_0: *name = "gemv<q4_0>"; break;
        case kQ4_1: *name = "gemv<q4_1>"; break;
        case kQ5_0: *name = "gemv<q5_0>"; break;
        case kQ5_1: *name = "gemv<q5_1>"; break;
        default: return hipErrorInvalidValue;
    }
    int64_t row_bytes = (K / block_values_of(type)) * layout.stride;
    int n = int(N), k = int(K), stride = layout.stride, off = layout.off;
    void* args[] = {&W, &x, &y, &n, &k, &row_bytes, &tile, &stride, &off};
    return hipLaunchKernel(kern, dim3(grid), dim3(kGemvThreads), args, shmem, s);
}

}  // namespace mq
