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
// scale.  Q4_K also needs the f32 sum of x over each 32-block (min term); Q6_K
// the sum over each 16-value run (code offset 32).
#include <cstdio>
#include <cstdlib>

#include "mq_device.h"
#include "mq_internal.h"

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

struct Stage {
    const uint32_t* p0;   // digit planes, 4 values per dword
    const uint32_t* p1;
    const uint32_t* p2;
    const int* ex;        // block exponent e_b (x = 2^e_b * v)
    const float* sum32;   // f32 sum of x per 32-block (Q4_K)
    const float* sum16;   // f32 sum of x per 16-value run (Q6_K)
};

// ---------------------------------------------------------------- Q4_K
// Unit u of a row: super-block u/4, 64-value group c = u%4 (sub-blocks 2c and
// 2c+1).  Bytes: 16-byte header (d, dmin, packed scales) and the 32 code bytes
// at 16 + 32c; byte i holds the code of value 64c+i (low nibble) and of value
// 64c+32+i (high nibble).
struct UnitQ4K {
    static constexpr int kValues = 64;
    uint4 hd, q0, q1;

    __device__ void load(const uint8_t* __restrict__ row, int u) {
        const uint8_t* blk = row + 144 * (u >> 2);
        hd = *reinterpret_cast<const uint4*>(blk);
        const uint4* qs = reinterpret_cast<const uint4*>(blk + 16 + 32 * (u & 3));
        q0 = qs[0];
        q1 = qs[1];
    }

    // exact dot of 32 codes (8 dwords) with the 32 staged values starting at dword w0
    __device__ static int run_dot(const uint32_t (&c)[8], const Stage& st, int w0) {
        const uint4* a = reinterpret_cast<const uint4*>(st.p0 + w0);
        const uint4* b = reinterpret_cast<const uint4*>(st.p1 + w0);
        const uint4* e = reinterpret_cast<const uint4*>(st.p2 + w0);
        int s0 = 0, s1 = 0, s2 = 0;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint4 x0 = a[k], x1 = b[k], x2 = e[k];
            s0 = sdot4(c[4 * k + 0], x0.x, s0); s0 = sdot4(c[4 * k + 1], x0.y, s0);
            s0 = sdot4(c[4 * k + 2], x0.z, s0); s0 = sdot4(c[4 * k + 3], x0.w, s0);
            s1 = sdot4(c[4 * k + 0], x1.x, s1); s1 = sdot4(c[4 * k + 1], x1.y, s1);
            s1 = sdot4(c[4 * k + 2], x1.z, s1); s1 = sdot4(c[4 * k + 3], x1.w, s1);
            s2 = sdot4(c[4 * k + 0], x2.x, s2); s2 = sdot4(c[4 * k + 1], x2.y, s2);
            s2 = sdot4(c[4 * k + 2], x2.z, s2); s2 = sdot4(c[4 * k + 3], x2.w, s2);
        }
        // |s2| <= 32 * 15 * 32, so the int32 combination cannot overflow
        return (s2 << 16) + (s1 << 8) + s0;
    }

    __device__ float dot(const Stage& st, int u) const {
        const int c = u & 3;
        const int blk0 = 8 * (u >> 2) + 2 * c;   // 32-block index of sub-block 2c
        const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        uint32_t lo[8], hi[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            lo[k] = w[k] & 0x0F0F0F0Fu;
            hi[k] = (w[k] >> 4) & 0x0F0F0F0Fu;
        }
        const int ilo = run_dot(lo, st, 8 * blk0);
        const int ihi = run_dot(hi, st, 8 * blk0 + 8);
        const float d = half_bits_to_float(hd.x & 0xFFFFu);
        const float dmin = half_bits_to_float(hd.x >> 16);
        uint32_t sc0, m0, sc1, m1;
        q4k_scale_min(hd.y, hd.z, hd.w, 2 * c, sc0, m0);
        q4k_scale_min(hd.y, hd.z, hd.w, 2 * c + 1, sc1, m1);
        const float codes = ldexpf(float(sc0) * float(ilo), st.ex[blk0]) +
                            ldexpf(float(sc1) * float(ihi), st.ex[blk0 + 1]);
        const float mins = fmaf(float(m0), st.sum32[blk0], float(m1) * st.sum32[blk0 + 1]);
        return fmaf(d, codes, -dmin * mins);
    }
};

// ---------------------------------------------------------------- Q6_K
// Unit u: super-block u/4, half h = (u/2)%2, lane run l in [l0, l0+16) with
// l0 = 16*(u%2): values 128h + 32t + l for t < 4 (16 each, one sub-scale each).
// Low 4 bits: ql[64h + l] (t = 0 low nibble, t = 2 high nibble) and
// ql[64h + 32 + l] (t = 1, 3); high 2 bits: bits 2t..2t+1 of qh[32h + l].
// Blocks are 210 bytes, so a block starts on a 2-byte boundary: every segment
// is read as naturally aligned dwords and realigned with v_alignbyte.
struct UnitQ6K {
    static constexpr int kValues = 64;
    uint32_t a[5], b[5], hq[5], s[3];
    uint32_t dbits;
    uint32_t shift;

    __device__ void load(const uint8_t* __restrict__ row, int u) {
        const uint8_t* blk = row + 210 * (u >> 2);
        const int h = (u >> 1) & 1, l0 = 16 * (u & 1);
        const uintptr_t base = reinterpret_cast<uintptr_t>(blk);
        shift = uint32_t(base & 3);
        const uint32_t* p = reinterpret_cast<const uint32_t*>(base & ~uintptr_t(3));
        // Every dword read holds at least one byte of this block, so none can
        // fault: segments end at most 196 bytes in, the scales end at 210.
        const uint32_t* pa = p + (64 * h + l0) / 4;
        const uint32_t* pb = p + (64 * h + 32 + l0) / 4;
        const uint32_t* ph = p + (128 + 32 * h + l0) / 4;
        const uint32_t* ps = p + (192 + 8 * h) / 4;
#pragma unroll
        for (int i = 0; i < 5; ++i) { a[i] = pa[i]; b[i] = pb[i]; hq[i] = ph[i]; }
#pragma unroll
        for (int i = 0; i < 3; ++i) s[i] = ps[i];
        dbits = load_u16(blk + 208);
    }

    __device__ float dot(const Stage& st, int u) const {
        const int h = (u >> 1) & 1, hi16 = u & 1, l0 = 16 * hi16;
        const int base = 256 * (u >> 2) + 128 * h + l0;   // value index of t = 0, l = l0
        uint32_t A[4], B[4], H[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            A[i] = align_byte(a[i + 1], a[i], shift);
            B[i] = align_byte(b[i + 1], b[i], shift);
            H[i] = align_byte(hq[i + 1], hq[i], shift);
        }
        const uint32_t s0 = align_byte(s[1], s[0], shift), s1 = align_byte(s[2], s[1], shift);
        float acc = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int v0 = base + 32 * t;               // 16 values v0 .. v0+15
            const uint4 x0 = *reinterpret_cast<const uint4*>(st.p0 + (v0 >> 2));
            const uint4 x1 = *reinterpret_cast<const uint4*>(st.p1 + (v0 >> 2));
            const uint4 x2 = *reinterpret_cast<const uint4*>(st.p2 + (v0 >> 2));
            const uint32_t xs0[4] = {x0.x, x0.y, x0.z, x0.w};
            const uint32_t xs1[4] = {x1.x, x1.y, x1.z, x1.w};
            const uint32_t xs2[4] = {x2.x, x2.y, x2.z, x2.w};
            int d0 = 0, d1 = 0, d2 = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t ql = (t & 1) ? B[i] : A[i];
                const uint32_t lo = (t < 2) ? ql : (ql >> 4);
                const uint32_t hb = (H[i] >> (2 * t)) & 0x03030303u;
                const uint32_t code = (lo & 0x0F0F0F0Fu) | (hb << 4);   // bytes: codes 0..63
                d0 = sdot4(code, xs0[i], d0);
                d1 = sdot4(code, xs1[i], d1);
                d2 = sdot4(code, xs2[i], d2);
            }
            // sum((c - 32) * x) = 2^e * sum(c * v) - 32 * sum(x)
            const float cv = ldexpf(combine3(d2, d1, d0), st.ex[v0 >> 5]);
            const int g = 2 * t + hi16;                  // sub-scale byte within this half
            const uint32_t word = g < 4 ? s0 : s1;
            const float sc = float(int32_t(word << (24 - 8 * (g & 3))) >> 24);
            acc = fmaf(sc, fmaf(-32.0f, st.sum16[v0 >> 4], cv), acc);
        }
        return half_bits_to_float(dbits) * acc;
    }
};

// ---------------------------------------------------------------- Q8_0
// Unit u = block u (34 bytes: f16 d, 32 int8 codes), 2-byte aligned.
struct UnitQ80 {
    static constexpr int kValues = 32;
    uint32_t w[9];
    uint32_t odd;

    __device__ void load(const uint8_t* __restrict__ row, int u) {
        const uintptr_t base = reinterpret_cast<uintptr_t>(row + 34 * u);
        odd = uint32_t(base & 2);
        const uint32_t* p = reinterpret_cast<const uint32_t*>(base & ~uintptr_t(3));
        // 9 naturally aligned dwords cover the block; each holds a byte of it
#pragma unroll
        for (int i = 0; i < 9; ++i) w[i] = p[i];
    }

    __device__ float dot(const Stage& st, int u) const {
        const float d = half_bits_to_float(odd ? (w[0] >> 16) : (w[0] & 0xFFFFu));
        const uint4* a = reinterpret_cast<const uint4*>(st.p0 + 8 * u);
        const uint4* b = reinterpret_cast<const uint4*>(st.p1 + 8 * u);
        const uint4* e = reinterpret_cast<const uint4*>(st.p2 + 8 * u);
        int s0 = 0, s1 = 0, s2 = 0;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint4 x0 = a[k], x1 = b[k], x2 = e[k];
            const uint32_t xs0[4] = {x0.x, x0.y, x0.z, x0.w};
            const uint32_t xs1[4] = {x1.x, x1.y, x1.z, x1.w};
            const uint32_t xs2[4] = {x2.x, x2.y, x2.z, x2.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int i = 4 * k + j;
                const uint32_t c = odd ? w[i + 1] : align_byte(w[i + 1], w[i], 2);
                s0 = sdot4(c, xs0[j], s0);
                s1 = sdot4(c, xs1[j], s1);
                s2 = sdot4(c, xs2[j], s2);
            }
        }
        return d * ldexpf(combine3(s2, s1, s0), st.ex[u]);
    }
};

template <int QT> struct UnitOf;
template <> struct UnitOf<kQ4_K> { using T = UnitQ4K; };
template <> struct UnitOf<kQ6_K> { using T = UnitQ6K; };
template <> struct UnitOf<kQ8_0> { using T = UnitQ80; };

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

// LDS layout (dynamic): planes 3 x K bytes | block exponents int [K/32] |
// sums f32 [K/32] (Q4_K) or [K/16] (Q6_K) | partials f32 [tile_units]
template <int QT, int kThreads, int kSlots>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const uint8_t* __restrict__ W,
                                                        const float* __restrict__ x,
                                                        float* __restrict__ y, int N, int K,
                                                        int64_t row_bytes, int tile_units) {
    using Unit = typename UnitOf<QT>::T;
    extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
    uint32_t* p0 = smem;
    uint32_t* p1 = p0 + (K >> 2);
    uint32_t* p2 = p1 + (K >> 2);
    int* ex = reinterpret_cast<int*>(p2 + (K >> 2));
    float* sums = reinterpret_cast<float*>(ex + (K >> 5));
    float* part = sums + (QT == kQ6_K ? (K >> 4) : (QT == kQ4_K ? (K >> 5) : 0));

    const int tid = threadIdx.x;
    const int U = K / Unit::kValues;
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

    Unit buf[kSlots];
    Cursor ld, cp;
    int t0 = r_begin;
    auto prime = [&](int tfirst) {
        const int units = min(rows_per_tile, r_end - tfirst) * U;
        const uint8_t* tile = W + int64_t(tfirst) * row_bytes;
        start(ld, tile);
        start(cp, tile);
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
            if (ld.f < units) buf[j].load(ld.row, ld.u);
            advance(ld);
        }
    };
    // Issue the first tile's weight loads before staging x.
    prime(t0);

    // Stage x: 8 lanes per 32-block, 4 values (one float4) per lane.
    for (int i = tid; i < (K >> 2); i += kThreads) {
        const float4 v = reinterpret_cast<const float4*>(x)[i];
        float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        a = fmaxf(a, __shfl_xor(a, 1, 64));
        a = fmaxf(a, __shfl_xor(a, 2, 64));
        a = fmaxf(a, __shfl_xor(a, 4, 64));
        // amax = m * 2^E, m in [0.5, 1): scale by 2^(21 - E) puts the block in [2^20, 2^21)
        const int k = kFracBits - __builtin_amdgcn_frexp_expf(a);
        uint32_t d0, d1, d2;
        transpose_digits(digits(v.x, k), digits(v.y, k), digits(v.z, k), digits(v.w, k), d0, d1, d2);
        p0[i] = d0;
        p1[i] = d1;
        p2[i] = d2;
        float s = (v.x + v.y) + (v.z + v.w);
        if constexpr (QT == kQ6_K) {
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            if ((i & 3) == 0) sums[i >> 2] = s;
        } else if constexpr (QT == kQ4_K) {
            s += __shfl_xor(s, 1, 64);
            s += __shfl_xor(s, 2, 64);
            s += __shfl_xor(s, 4, 64);
            if ((i & 7) == 0) sums[i >> 3] = s;
        }
        if ((i & 7) == 0) ex[i >> 3] = -k;
    }
    __syncthreads();

    const Stage st{p0, p1, p2, ex, sums, sums};

    for (; t0 < r_end; t0 += rows_per_tile) {
        const int rows = min(rows_per_tile, r_end - t0);
        const int units = rows * U;

        for (int base = 0; base < units; base += kSlots * kThreads) {
#pragma unroll
            for (int j = 0; j < kSlots; ++j) {
                if (cp.f < units) {
                    part[cp.f] = buf[j].dot(st, cp.u);
                    advance(cp);
                    if (ld.f < units) buf[j].load(ld.row, ld.u);
                    advance(ld);
                }
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

size_t fixed_lds_bytes(int type, int64_t K) {
    size_t b = size_t(K) * 3 + size_t(K / 32) * 4;
    if (type == kQ4_K) b += size_t(K / 32) * 4;
    if (type == kQ6_K) b += size_t(K / 16) * 4;
    return b;
}

// Threads per workgroup and ring depth, per type; an MQ_GEMV_CONFIG=threads,slots
// environment setting (read once, bench A/B only) picks another built variant.
struct Config {
    int threads, slots;
};
constexpr Config kConfigs[] = {{1024, 2}, {1024, 3}, {1024, 4}, {512, 4}, {512, 6}, {512, 8}};

template <int QT, int T, int S>
const void* kernel_ptr() {
    return reinterpret_cast<const void*>(gemv_kernel<QT, T, S>);
}

template <int QT>
const void* pick_kernel(Config c) {
    if (c.threads == 1024 && c.slots == 2) return kernel_ptr<QT, 1024, 2>();
    if (c.threads == 1024 && c.slots == 3) return kernel_ptr<QT, 1024, 3>();
    if (c.threads == 1024 && c.slots == 4) return kernel_ptr<QT, 1024, 4>();
    if (c.threads == 512 && c.slots == 4) return kernel_ptr<QT, 512, 4>();
    if (c.threads == 512 && c.slots == 6) return kernel_ptr<QT, 512, 6>();
    if (c.threads == 512 && c.slots == 8) return kernel_ptr<QT, 512, 8>();
    return nullptr;
}

const void* kernel_for(int type, Config c) {
    switch (type) {
        case kQ4_K: return pick_kernel<kQ4_K>(c);
        case kQ6_K: return pick_kernel<kQ6_K>(c);
        case kQ8_0: return pick_kernel<kQ8_0>(c);
        default: return nullptr;
    }
}

Config default_config(int type) {
    switch (type) {
        case kQ4_K: return {1024, 2};
        case kQ6_K: return {1024, 2};
        default: return {1024, 2};
    }
}

Config chosen_config(int type) {
    static int env_threads = -1, env_slots = -1;
    if (env_threads < 0) {
        env_threads = 0;
        env_slots = 0;
        if (const char* e = getenv("MQ_GEMV_CONFIG")) {
            int t = 0, s = 0;
            if (sscanf(e, "%d,%d", &t, &s) == 2) { env_threads = t; env_slots = s; }
        }
    }
    if (env_threads > 0) {
        const Config c{env_threads, env_slots};
        if (kernel_for(type, c)) return c;
    }
    return default_config(type);
}

}  // namespace

// Largest tile (in units) that fits next to the staged x; 0 if not even one row fits.
int gemv_tile_units(int type, int64_t K, size_t lds_limit) {
    const size_t fixed = fixed_lds_bytes(type, K);
    const int vals = type == kQ8_0 ? 32 : 64;
    const int64_t U = K / vals;
    if (lds_limit <= fixed) return 0;
    int64_t units = int64_t((lds_limit - fixed) / 4);
    if (units > 65536) units = 65536;
    if (units < U) return 0;
    return int(units);
}

hipError_t gemv_set_attributes(size_t lds_limit) {
    for (int type : {kQ4_K, kQ6_K, kQ8_0}) {
        for (const Config& c : kConfigs) {
            hipError_t e = hipFuncSetAttribute(kernel_for(type, c), hipFuncAttributeMaxDynamicSharedMemorySize,
                                               int(lds_limit));
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

hipError_t launch_gemv(int type, const uint8_t* W, const float* x, float* y, int64_t N, int64_t K,
                       hipStream_t s, const char** name) {
    const DeviceInfo* info = device_info();
    if (!info) return hipErrorInvalidDevice;
    int tile = gemv_tile_units(type, K, info->lds_per_block);
    if (tile <= 0) return hipErrorInvalidValue;
    const int vals = type == kQ8_0 ? 32 : 64;
    const int U = int(K / vals);
    // Rows of one workgroup; shrink the tile so a workgroup's rows split into equal tiles.
    const int grid = int(N < info->cu_count ? N : info->cu_count);
    const int64_t rows_wg = (N + grid - 1) / grid;
    const int64_t max_rows = tile / U;
    const int64_t ntiles = (rows_wg + max_rows - 1) / max_rows;
    const int64_t rows_tile = (rows_wg + ntiles - 1) / ntiles;
    tile = int(rows_tile * U);
    const size_t shmem = fixed_lds_bytes(type, K) + size_t(tile) * 4;
    const Config c = chosen_config(type);
    const void* kern = kernel_for(type, c);
    int64_t row_bytes = 0;
    switch (type) {
        case kQ8_0: *name = "gemv<q8_0>"; row_bytes = (K / 32) * 34; break;
        case kQ4_K: *name = "gemv<q4_K>"; row_bytes = (K / 256) * 144; break;
        case kQ6_K: *name = "gemv<q6_K>"; row_bytes = (K / 256) * 210; break;
        default: return hipErrorInvalidValue;
    }
    int n = int(N), k = int(K);
    void* args[] = {&W, &x, &y, &n, &k, &row_bytes, &tile};
    return hipLaunchKernel(kern, dim3(grid), dim3(c.threads), args, shmem, s);
}

}  // namespace mq
