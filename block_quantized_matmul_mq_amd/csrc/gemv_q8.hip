// mq_gemm for a few activation rows (M <= 8): a multi-row GEMV over the quantized
// activation plane ("minfer CUDA Backend Design", 4.4 Execution dispatch: the int8
// product over q8 activation blocks; a handful of rows is a matrix-vector product per
// row that should read every weight byte once for all of them).
//
// Work split and weight stream as in the f32-x GEMV (gemv.hip): one 1024-thread
// workgroup per CU owns a contiguous range of rows, cut into units (64 values for Q4_K
// and Q6_K, one 32-value block for Q8_0) dealt round-robin to the lanes, each lane
// loading its next units while it computes the current one.  A unit's weight bytes are
// read once and meet all MR activation rows.
//
// Activation.  The workgroup stages the M rows' int8 codes in LDS, one plane per row in
// the unit-major chunk layout of gemv.hip (conflict-free 16-byte reads), rows M..MR-1
// zero, with per-(row, unit) factors: the block scales dx (and, for Q4_K, dx times the
// block's code sum, which carries the min term; for Q6_K, 32 times the code sum of each
// 16-value run, which turns the unsigned code c into c - 32).
//
// Per unit and row the block dots are exact int32 sums of v_dot4_i32_i8 (code x q8
// code), scaled in f32:
//   Q4_K: d sc_j dx_j D_j - dmin m_j dx_j S_j   (two 32-value sub-blocks j)
//   Q6_K: d s_t dx_t (D_t - 32 S_t)              (four 16-value runs t)
//   Q8_0: d dx D
// Lane partials go to LDS, [unit][row]; each output is summed over its row's units in
// a fixed order (deterministic).  With DUMP the kernel also writes the int32 block dots
// (the test export of mq_debug_gemm_blockdots).
#include <cstdint>
#include <type_traits>

#include "mq_device.h"
#include "mq_internal.h"
#include "weight_units.h"

namespace mq {

namespace {

constexpr int kThreads = 1024;
constexpr int kSlots = 2;

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4(int(a), int(b), c, false);
}

// dot of 16 codes (4 dwords) with 16 activation codes (one 16-byte chunk)
__device__ __forceinline__ int dot16(const uint32_t* c, const uint4& x, int s) {
    s = sdot4(c[0], x.x, s);
    s = sdot4(c[1], x.y, s);
    s = sdot4(c[2], x.z, s);
    return sdot4(c[3], x.w, s);
}

template <int QT> struct Shape;
template <> struct Shape<kQ4_K> { static constexpr int kValues = 64, kChunks = 4; };
template <> struct Shape<kQ6_K> { static constexpr int kValues = 64, kChunks = 4; };
template <> struct Shape<kQ8_0> { static constexpr int kValues = 32, kChunks = 2; };
template <> struct Shape<kQ5_K> { static constexpr int kValues = 64, kChunks = 4; };
template <> struct Shape<kQ4_0> { static constexpr int kValues = 32, kChunks = 2; };
template <> struct Shape<kQ4_1> { static constexpr int kValues = 32, kChunks = 2; };
template <> struct Shape<kQ5_0> { static constexpr int kValues = 32, kChunks = 2; };
template <> struct Shape<kQ5_1> { static constexpr int kValues = 32, kChunks = 2; };

template <int QT> struct UnitT { using T = RawLegacy<QT>; };
template <> struct UnitT<kQ4_K> { using T = RawQ4K; };
template <> struct UnitT<kQ5_K> { using T = RawQ5K; };
template <> struct UnitT<kQ6_K> { using T = RawQ6K; };
template <> struct UnitT<kQ8_0> { using T = RawQ80; };

// Per-(row, unit) activation factors: the 32-value types keep the block scale and the
// block's code sum (their offset or min term needs it exactly).
struct ScaleSum {
    float dx;
    int32_t S;
};

// unit and chunk of the 16 values starting at `val` (a multiple of 16) -- the layouts of
// the units in weight_units.h
template <int QT>
__device__ __forceinline__ void unit_chunk(int val, int& uu, int& kc) {
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
}

// LDS (dynamic): MR code planes of kChunks * S * 16 bytes (S = U + 1) | per-row factors
// (Q4_K, Q5_K: float4 [MR][U]; Q6_K: float4 [MR][U] then int4 [MR][U]; Q8_0: float [MR][U];
// the 32-value types: ScaleSum [MR][U]) | partials f32 [tile_units][MR].
__host__ __device__ constexpr size_t factor_unit_bytes(int type) {
    return (type == kQ4_K || type == kQ5_K) ? 16 : (type == kQ6_K ? 32 : (type == kQ8_0 ? 4 : 8));
}
template <int QT, int MR>
__host__ __device__ constexpr size_t factor_bytes(int U) {
    return size_t(MR) * U * factor_unit_bytes(QT);
}

template <int QT, int MR, bool DUMP>
__global__ __launch_bounds__(kThreads) void gemv_q8_kernel(const uint8_t* __restrict__ W,
                                                           const int8_t* __restrict__ codes,
                                                           const float* __restrict__ xscale,
                                                           const int32_t* __restrict__ xsum, float* __restrict__ Y,
                                                           int32_t* __restrict__ dots, int M, int N, int K,
                                                           int64_t row_bytes, int tile_units, int blk_stride,
                                                           int blk_off) {
    using Sh = Shape<QT>;
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const int U = K / Sh::kValues;
    const int S = U + 1;
    const int plane = Sh::kChunks * S * 16;
    const int KB = K >> 5;
    uint8_t* planes = smem;
    uint8_t* fac = planes + MR * plane;
    float* part = reinterpret_cast<float*>(fac + factor_bytes<QT, MR>(U));

    const int tid = threadIdx.x;
    const int r_begin = int((int64_t(blockIdx.x) * N) / gridDim.x);
    const int r_end = int((int64_t(blockIdx.x + 1) * N) / gridDim.x);
    const int rows_per_tile = max(1, tile_units / U);

    using Unit = typename UnitT<QT>::T;
    // A lane handles flat unit indices f = tid, tid + kThreads, ... of a tile; two cursors
    // (next load, next compute) step by kThreads units without multiplies or divisions.
    const int dq = kThreads / U, dr = kThreads - dq * U;
    const int64_t dq_bytes = int64_t(dq) * row_bytes;
    struct Cursor {
        int f, u, r;            // unit of the tile, unit of the row, row of the tile
        const uint8_t* row;
    };
    auto start = [&](Cursor& c, const uint8_t* tile) {
        c.f = tid;
        c.r = tid / U;
        c.u = tid - c.r * U;
        c.row = tile + int64_t(c.r) * row_bytes;
    };
    auto advance = [&](Cursor& c) {
        c.f += kThreads;
        c.u += dr;
        c.r += dq;
        c.row += dq_bytes;
        if (c.u >= U) {
            c.u -= U;
            ++c.r;
            c.row += row_bytes;
        }
    };

    // Weight ring: kSlots units ahead of the compute (as in gemv.hip: the steady loop issues
    // every load, a dead lane of a tile's last round re-reads the tile's first unit).
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
    prime(t0);

    // Stage the activation rows: 16-byte chunks of codes to their (unit, chunk) slots.
    const int nchunks = K >> 4;
    for (int i = tid; i < MR * nchunks; i += kThreads) {
        const int m = i / nchunks, c16 = i - m * nchunks;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (m < M) v = *reinterpret_cast<const uint4*>(codes + int64_t(m) * K + 16 * c16);
        int uu, kc;
        unit_chunk<QT>(16 * c16, uu, kc);
        *reinterpret_cast<uint4*>(planes + m * plane + (kc * S + uu) * 16) = v;
        if constexpr (QT == kQ6_K) {   // 32 x the run's code sum (c16 is run kc of unit uu)
            int s = sdot4(v.x, 0x01010101u, 0);
            s = sdot4(v.y, 0x01010101u, s);
            s = sdot4(v.z, 0x01010101u, s);
            s = sdot4(v.w, 0x01010101u, s);
            reinterpret_cast<int*>(fac + size_t(MR) * U * 16)[(m * U + uu) * 4 + kc] = 32 * s;
        }
    }
    // Per-(row, unit) block factors.
    for (int i = tid; i < MR * U; i += kThreads) {
        const int m = i / U, uu = i - m * U;
        const bool live = m < M;
        const float* xs = xscale + int64_t(m) * KB;
        if constexpr (QT == kQ4_K || QT == kQ5_K) {
            float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
            if (live) {
                const int32_t* su = xsum + int64_t(m) * KB;
                const float d0 = xs[2 * uu], d1 = xs[2 * uu + 1];
                f = make_float4(d0, d1, d0 * float(su[2 * uu]), d1 * float(su[2 * uu + 1]));
            }
            reinterpret_cast<float4*>(fac)[i] = f;
        } else if constexpr (QT == kQ6_K) {
            // run t of unit uu lies in 32-block 8 (uu / 4) + 4 h + t, h = (uu / 2) % 2
            float4 f = make_float4(0.f, 0.f, 0.f, 0.f);
            if (live) {
                const int b0 = 8 * (uu >> 2) + 4 * ((uu >> 1) & 1);
                f = make_float4(xs[b0], xs[b0 + 1], xs[b0 + 2], xs[b0 + 3]);
            }
            reinterpret_cast<float4*>(fac)[i] = f;
        } else if constexpr (QT == kQ8_0) {
            reinterpret_cast<float*>(fac)[i] = live ? xs[uu] : 0.f;
        } else {
            reinterpret_cast<ScaleSum*>(fac)[i] = live ? ScaleSum{xs[uu], xsum[int64_t(m) * KB + uu]} : ScaleSum{0.f, 0};
        }
    }
    __syncthreads();

    // One unit against the MR rows: r[m] = this unit's share of Y[m][row].
    auto dot = [&](const Unit& w, int uu, int row, float (&r)[MR]) {
        auto chunk = [&](int m, int kc) {
            return *reinterpret_cast<const uint4*>(planes + m * plane + (kc * S + uu) * 16);
        };
        if constexpr (QT == kQ4_K || QT == kQ5_K) {
            uint32_t lo[8], hi[8], scp, mnp;
            if constexpr (QT == kQ4_K) w.codes(lo, hi);
            else w.codes(uu, lo, hi);
            w.scale_min(uu & 3, scp, mnp);
            const float d = w.d(), dmin = w.dmin();
            const float a0 = d * ubyte_f<0>(scp), a1 = d * ubyte_f<1>(scp);
            const float b0 = dmin * ubyte_f<0>(mnp), b1 = dmin * ubyte_f<1>(mnp);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const int Dlo = dot16(lo + 4, chunk(m, 1), dot16(lo, chunk(m, 0), 0));
                const int Dhi = dot16(hi + 4, chunk(m, 3), dot16(hi, chunk(m, 2), 0));
                const float4 f = reinterpret_cast<const float4*>(fac)[m * U + uu];
                r[m] = fmaf(a0 * f.x, float(Dlo), fmaf(a1 * f.y, float(Dhi), -fmaf(b0, f.z, b1 * f.w)));
                if constexpr (DUMP) {
                    int32_t* o = dots + (int64_t(m) * N + row) * KB + 2 * uu;
                    if (m < M) {
                        o[0] = Dlo;
                        o[1] = Dhi;
                    }
                }
            }
        } else if constexpr (QT == kQ6_K) {
            uint32_t A[4], B[4], H[4], s0, s1, code[4][4];
            w.realign(A, B, H, s0, s1);
            const float d = w.d();
            float sc[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                RawQ6K::run_codes(t, A, B, H, code[t]);
                sc[t] = d * RawQ6K::subscale(t, uu, s0, s1);
            }
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const float4 f = reinterpret_cast<const float4*>(fac)[m * U + uu];
                const int4 s32 = reinterpret_cast<const int4*>(fac + size_t(MR) * U * 16)[m * U + uu];
                const float fv[4] = {f.x, f.y, f.z, f.w};
                const int sv[4] = {s32.x, s32.y, s32.z, s32.w};
                float acc = 0.f;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int D = dot16(code[t], chunk(m, t), 0) - sv[t];   // sum (c - 32) q, exact
                    acc = fmaf(sc[t] * fv[t], float(D), acc);
                    if constexpr (DUMP) {
                        // group g = 16-value group index along the row: unit uu, run t
                        const int g = 16 * (uu >> 2) + 8 * ((uu >> 1) & 1) + 2 * t + (uu & 1);
                        if (m < M) dots[(int64_t(m) * N + row) * (K >> 4) + g] = D;
                    }
                }
                r[m] = acc;
            }
        } else if constexpr (QT == kQ8_0) {
            uint32_t c[8];
            w.codes(c);
            const float d = w.d();
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const int D = dot16(c + 4, chunk(m, 1), dot16(c, chunk(m, 0), 0));
                r[m] = d * reinterpret_cast<const float*>(fac)[m * U + uu] * float(D);
                if constexpr (DUMP) {
                    if (m < M) dots[(int64_t(m) * N + row) * KB + uu] = D;
                }
            }
        } else {
            // Q4_0 / Q5_0: the block dot of (code - offset), exact: D - offset * S.
            // Q4_1 / Q5_1: d * dx * D + m * dx * S.
            uint32_t c[8];
            w.codes(c);
            const float d = w.d();
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                const int D = dot16(c + 4, chunk(m, 1), dot16(c, chunk(m, 0), 0));
                const ScaleSum f = reinterpret_cast<const ScaleSum*>(fac)[m * U + uu];
                int E = D;
                if constexpr (Legacy<QT>::kMin) {
                    r[m] = fmaf(d * f.dx, float(D), w.m() * (f.dx * float(f.S)));
                } else {
                    E = D - Legacy<QT>::kOffset * f.S;
                    r[m] = d * f.dx * float(E);
                }
                if constexpr (DUMP) {
                    if (m < M) dots[(int64_t(m) * N + row) * KB + uu] = E;
                }
            }
        }
    };
    auto compute = [&](const Unit& w, const Cursor& c) {
        if (c.f < units) {
            float r[MR];
            dot(w, c.u, t0 + c.r, r);
            float* p = part + int64_t(c.f) * MR;
#pragma unroll
            for (int m = 0; m < MR; ++m) p[m] = r[m];
        }
    };

    for (; t0 < r_end; t0 += rows_per_tile) {
        const int rows = min(rows_per_tile, r_end - t0);
        int it0 = 0;
        for (; it0 + 2 * kSlots <= iters; it0 += kSlots) {
#pragma unroll
            for (int j = 0; j < kSlots; ++j) {
                compute(buf[j], cp);
                advance(cp);
                load_next(j);
            }
        }
#pragma unroll
        for (int j = 0; j < 2 * kSlots; ++j) {
            if (it0 + j < iters) {
                compute(buf[j % kSlots], cp);
                advance(cp);
                if (it0 + j + kSlots < iters) load_next(j % kSlots);
            }
        }
        const int t1 = t0 + rows_per_tile;
        if (t1 < r_end) prime(t1);
        __syncthreads();

        // Y[m][t0 + row] = sum over the row's units, in unit order
        if constexpr (!DUMP) {
            for (int p = tid; p < rows * MR; p += kThreads) {
                const int row = p / MR, m = p - row * MR;
                if (m >= M) continue;
                const float* pr = part + int64_t(row) * U * MR + m;
                float s = 0.f;
                for (int j = 0; j < U; ++j) s += pr[j * MR];
                Y[int64_t(m) * N + t0 + row] = s;
            }
        }
        __syncthreads();
    }
}

size_t fixed_bytes(int type, int MR, int64_t K) {
    const int vals = unit_values(type), chunks = vals / 16;
    const int U = int(K / vals);
    const size_t planes = size_t(MR) * chunks * (U + 1) * 16;
    return planes + size_t(MR) * U * factor_unit_bytes(type);
}

int rows_for(int64_t M) { return M <= 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : 8)); }

template <int QT, int MR>
const void* kernel_ptr(bool dump) {
    return dump ? reinterpret_cast<const void*>(gemv_q8_kernel<QT, MR, true>)
                : reinterpret_cast<const void*>(gemv_q8_kernel<QT, MR, false>);
}

template <int QT>
const void* kernel_for_type(int mr, bool dump) {
    switch (mr) {
        case 1: return kernel_ptr<QT, 1>(dump);
        case 2: return kernel_ptr<QT, 2>(dump);
        case 4: return kernel_ptr<QT, 4>(dump);
        default: return kernel_ptr<QT, 8>(dump);
    }
}

const void* kernel_for(int type, int mr, bool dump) {
    switch (type) {
        case kQ4_K: return kernel_for_type<kQ4_K>(mr, dump);
        case kQ5_K: return kernel_for_type<kQ5_K>(mr, dump);
        case kQ6_K: return kernel_for_type<kQ6_K>(mr, dump);
        case kQ8_0: return kernel_for_type<kQ8_0>(mr, dump);
        case kQ4_0: return kernel_for_type<kQ4_0>(mr, dump);
        case kQ4_1: return kernel_for_type<kQ4_1>(mr, dump);
        case kQ5_0: return kernel_for_type<kQ5_0>(mr, dump);
        case kQ5_1: return kernel_for_type<kQ5_1>(mr, dump);
        default: return nullptr;
    }
}

}  // namespace

bool gemv_q8_applies(int type, int64_t M, int64_t K) {
    // a function of the shape alone (the code planes, the factor arrays and the partials of
    // one row must fit the 160 KB of LDS a gfx950 workgroup may use), so that the scratch
    // sizing of mq_gemm does not depend on the device
    if (M < 1 || M > kGemvQ8MaxRows || !kernel_for(type, 1, false)) return false;
    const int mr = rows_for(M);
    return fixed_bytes(type, mr, K) + size_t(K / unit_values(type)) * mr * 4 <= kGfx950LdsBytes;
}

hipError_t gemv_q8_set_attributes(size_t lds_limit) {
    for (int type : {kQ4_K, kQ5_K, kQ6_K, kQ8_0, kQ4_0, kQ4_1, kQ5_0, kQ5_1})
        for (int mr : {1, 2, 4, 8})
            for (bool dump : {false, true}) {
                hipError_t e = hipFuncSetAttribute(kernel_for(type, mr, dump),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_limit));
                if (e != hipSuccess) return e;
            }
    return hipSuccess;
}

hipError_t launch_gemv_q8(int type, BlockLayout lay, const uint8_t* W, const int8_t* codes, const float* xs,
                          const int32_t* xsum, float* Y, int32_t* dots, int64_t M, int64_t N, int64_t K,
                          hipStream_t s, const char** name) {
    const DeviceInfo* info = device_info();
    if (!info) return hipErrorInvalidDevice;
    if (gemv_q8_tiled_applies(type, lay, W, codes, M, N, K, info->cu_count))
        return launch_gemv_q8_tiled(type, W, codes, xs, Y, dots, M, N, K, info->cu_count, s, name);
    const int mr = rows_for(M);
    const int vals = unit_values(type);
    const int U = int(K / vals);
    const size_t fixed = fixed_bytes(type, mr, K);
    if (fixed >= info->lds_per_block) return hipErrorInvalidValue;
    int64_t tile = int64_t((info->lds_per_block - fixed) / (size_t(mr) * 4));
    if (tile > 65536) tile = 65536;
    if (tile < U) return hipErrorInvalidValue;
    const int grid = int(N < info->cu_count ? N : info->cu_count);
    // rows of one workgroup split into equal tiles
    const int64_t rows_wg = (N + grid - 1) / grid;
    const int64_t max_rows = tile / U;
    const int64_t ntiles = (rows_wg + max_rows - 1) / max_rows;
    const int64_t rows_tile = (rows_wg + ntiles - 1) / ntiles;
    int tile_units = int(rows_tile * U);
    const size_t shmem = fixed + size_t(tile_units) * mr * 4;
    const bool repacked = lay.off != 0 || (type == kQ6_K && lay.stride != 210);
    switch (type) {
        case kQ8_0: *name = repacked ? "gemv_q8<q8_0 repacked>" : "gemv_q8<q8_0>"; break;
        case kQ4_K: *name = "gemv_q8<q4_K>"; break;
        case kQ5_K: *name = "gemv_q8<q5_K>"; break;
        case kQ6_K: *name = repacked ? "gemv_q8<q6_K repacked>" : "gemv_q8<q6_K>"; break;
        case kQ4_0: *name = "gemv_q8<q4_0>"; break;
        case kQ4_1: *name = "gemv_q8<q4_1>"; break;
        case kQ5_0: *name = "gemv_q8<q5_0>"; break;
        case kQ5_1: *name = "gemv_q8<q5_1>"; break;
        default: return hipErrorInvalidValue;
    }
    int64_t row_bytes = (K / block_values_of(type)) * lay.stride;
    int m = int(M), n = int(N), k = int(K), stride = lay.stride, off = lay.off;
    void* args[] = {&W, &codes, &xs, &xsum, &Y, &dots, &m, &n, &k, &row_bytes, &tile_units, &stride, &off};
    return hipLaunchKernel(kernel_for(type, mr, dots != nullptr), dim3(grid), dim3(kThreads), args, shmem, s);
}

}  // namespace mq
