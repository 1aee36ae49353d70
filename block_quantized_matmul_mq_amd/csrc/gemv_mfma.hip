// mq_gemv for wide Q4_K matrices and for Q4_K matrices with long rows: y = deq(W) x for
// one f32 activation row (the decode product of "minfer CUDA Backend Design", 4.4
// Execution dispatch), with the integer dot products on int8 matrix cores and the weights
// streamed through LDS.  The wide-matrix kernel is described first; the long-row kernel
// (more than 16 super-blocks per row, few rows per CU) further down.
//
// Work split.  The matrix is cut into tiles of 16 rows, dealt round-robin to the
// workgroups (one per CU): tile t goes to workgroup t % G, so at any moment the GPU reads
// one window of consecutive tiles (faster on HBM than one separate stream per CU).
// (Sharing the rows of the last, partial round out evenly, a partial tile per
// workgroup, was measured slower: a workgroup's time follows its item count.)
// Inside a workgroup, wave w owns super-block w of every row (rows of up to 16
// super-blocks, K <= 4096): its work item for a tile is that super-block of the tile's
// 16 rows, 16 x 144 bytes.  Each wave streams its own items into its own LDS ring of NB
// slots with buffer_load ... lds (16 consecutive bytes per lane, 9 lanes per 144-byte
// block) and waits only for its own loads, so the main loop has no workgroup barrier:
// a wave computes an item as soon as its bytes have landed, with NB - 1 items in flight.
//
// Activation.  x is staged once per workgroup in an exact integer form: per 32-value
// block b, x = 2^e_b * v with v = rint(x * 2^-e_b) of at most 21 bits (e_b puts the block
// maximum in [2^20, 2^21)); v is kept as three signed byte planes v = 65536 d2 + 256 d1 +
// d0.  Since a wave always sees the same super-block, it keeps that super-block's digits
// (the MFMA A operands), exponents and block sums in registers.
//
// Products.  v_mfma_i32_16x16x64_i8 on one item:
//   B (64 x 16): column n = row n of the tile; lane group q (lanes 16q .. 16q + 15) holds
//                16 codes of unit q (values 64q .. 64q + 63 of the super-block);
//   A (16 x 64): row 4q + p (p < 3) = digit plane p of the same 16 values in lane group q
//                and zero in the other groups; rows 4q + 3 are zero too.
// So C[4q + p][n] = exact sum over unit q's 16 values of code * d_p, and lane (n, q) gets
// exactly its own unit's three plane sums (C rows 4q .. 4q + 2 of column n).  Two MFMAs
// cover a 32-value sub-block (low nibbles: sub-block 2q, high nibbles: 2q + 1), four an
// item.  Each lane then applies its two sub-blocks' 6-bit scales and mins:
//   y[n] += d * sc * 2^e * sum(code * v) - dmin * m * sum(x)      (per sub-block).
// The four lanes of a row are summed with two lane swaps; each wave leaves one partial
// per row and tile in LDS, and at the end four lanes per row each add four of the row's
// wave partials and two lane swaps combine them (a fixed order: deterministic).
#include <utility>

#include "mq_device.h"
#include "mq_internal.h"

namespace mq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kTileRows = 16;
constexpr int kMaxSB = kWaves;                     // super-blocks per row: one per wave
constexpr int kMinSB = 12;                         // fewer leaves too many waves idle
constexpr int kItemBytes = kTileRows * 144;        // 2304: one super-block of 16 rows
constexpr int kFracBits = 21;
constexpr int kBufferWord3 = 0x00020000;           // raw buffer resource: 32-bit data format, no swizzle
constexpr int kStageBytes = 16384;                 // x staging, later the row partials
constexpr int kMaxTilesPerGroup = kStageBytes / (kTileRows * kWaves * 4);
static_assert(kMaxTilesPerGroup * kTileRows * 4 <= kThreads, "one pass of the row sums");

// f(integral_constant<int, 0>), ..., f(integral_constant<int, n - 1>)
template <class F, int... i>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, i...>) {
    (f(std::integral_constant<int, i>{}), ...);
}
template <int n, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, n>{});
}

// Wait until at most n vector memory operations of this wave are outstanding and its
// LDS operations are done, then a workgroup barrier.  (__syncthreads would also wait for
// every load in flight: its workgroup fence covers global memory.)  The "memory" clobber
// keeps the compiler from moving LDS accesses across it.
template <int n>
__device__ __forceinline__ void wait_barrier() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(n) : "memory");
}

// Byte k of four dwords -> one dword (a 4 x 4 byte transpose, three planes).
__device__ __forceinline__ void transpose3(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3, uint32_t& p0,
                                           uint32_t& p1, uint32_t& p2) {
    const uint32_t t01 = __builtin_amdgcn_perm(r1, r0, 0x05010400u);   // r0.b0 r1.b0 r0.b1 r1.b1
    const uint32_t t23 = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
    p0 = __builtin_amdgcn_perm(t23, t01, 0x05040100u);
    p1 = __builtin_amdgcn_perm(t23, t01, 0x07060302u);
    const uint32_t u01 = __builtin_amdgcn_perm(r1, r0, 0x00000602u);   // r0.b2 r1.b2
    const uint32_t u23 = __builtin_amdgcn_perm(r3, r2, 0x00000602u);
    p2 = __builtin_amdgcn_perm(u23, u01, 0x05040100u);
}

// Signed digits of v = rint(x * 2^k) (|v| <= 2^21) in bytes 0..2:
// (v + 0x808080) has unsigned bytes b_i = d_i + 128, and b_i ^ 0x80 is d_i as int8.
__device__ __forceinline__ uint32_t digits3(float x, int k) {
    const float f = ldexpf(x, k) + 12582912.0f;   // 1.5 * 2^23: the low mantissa bits are rint(x*2^k)
    return (__float_as_uint(f) - 0x4ABF7F80u) ^ 0x00808080u;
}

// The three digit-plane sums of a run as one int32: exact while |sum code * v| < 2^31, which
// holds for unsigned codes of up to 6 bits over runs of at most 16 values (16 * 63 * 2^21 <
// 2^31) and for Q4_K's 4-bit codes over 32 values.  Signed 8-bit codes (Q8_0) can reach
// 16 * 128 * 2^21 = 2^32 and take combine3f.
__device__ __forceinline__ int combine3(const v4i c) {
    return (((c[2] << 8) + c[1]) << 8) + c[0];
}
// The same sum in f32 (each plane sum is exact in int32; the combination is rounded once
// per term, f32-grade).
__device__ __forceinline__ float combine3f(const v4i c) {
    return fmaf(float(c[2]), 65536.0f, fmaf(float(c[1]), 256.0f, float(c[0])));
}

// Sum over the lanes l, l ^ 16, l ^ 32, l ^ 48 (v_permlane16_swap, v_permlane32_swap).
__device__ __forceinline__ float sum_lane_groups(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// NB: LDS ring slots per wave (items in flight + the one being computed).
template <int NB>
__global__ __launch_bounds__(kThreads) void gemv_mfma_q4k_kernel(const uint8_t* __restrict__ W,
                                                                 const float* __restrict__ x,
                                                                 float* __restrict__ y, int N, int K,
                                                                 int row_bytes) {
    // One static array per ring slot: with compile-time slot numbers the compiler knows
    // which slot a read touches and waits for that slot's loads only.
    __shared__ __attribute__((aligned(16))) uint8_t ring0[kWaves * kItemBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[kWaves * kItemBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ring2[NB > 2 ? kWaves * kItemBytes : 16];
    __shared__ __attribute__((aligned(16))) uint8_t ring3[NB > 3 ? kWaves * kItemBytes : 16];
    // x staging (digit planes [3][K], block exponents, block sums), then row partials
    // [tile][row][wave]: a barrier separates the last read of the one from the first
    // write of the other.
    __shared__ __attribute__((aligned(16))) uint8_t stage_lds[kStageBytes];
    auto slot = [&](auto b) -> uint8_t* {
        constexpr int B = decltype(b)::value;
        if constexpr (B == 0) return ring0;
        else if constexpr (B == 1) return ring1;
        else if constexpr (B == 2) return ring2;
        else return ring3;
    };
    int8_t* xp = reinterpret_cast<int8_t*>(stage_lds);
    int* ex = reinterpret_cast<int*>(stage_lds + 3 * 256 * kMaxSB);
    float* sums = reinterpret_cast<float*>(ex + 8 * kMaxSB);
    float* part = reinterpret_cast<float*>(stage_lds);

    const int SB = K >> 8;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x, w0 = blockIdx.x;
    const int TB = kTileRows * row_bytes;
    const int T = (N + kTileRows - 1) / kTileRows;
    const int tiles = (T - w0 + G - 1) / G;   // this workgroup's: global tiles w0 + k G
    const bool active = wave < SB;            // uniform: waves past the row's super-blocks only stage x

    // x first: loads complete in issue order, so x is requested before the weights.
    const int nquads = K >> 2;
    float4 xe = {};
    if (tid < nquads) xe = reinterpret_cast<const float4*>(x)[tid];

    // The matrix as one buffer: rows past the last (the last tile's tail, tiles past the
    // end) read as zeros through the buffer range check.
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W), 0, N * row_bytes, kBufferWord3);
    // This wave's item of a tile: 144 16-byte chunks c (row c / 9, bytes 16 (c % 9) of the
    // row's super-block), to slot bytes 16 c: chunks 0..63 and 64..127 with 16-byte lanes,
    // chunks 128..143 with 4-byte lanes.
    // Idle waves issue the same loads (so that every wave runs the same load sequence and
    // the compiler's wait counts stay exact), all past the end of the buffer: they move no
    // data (offsets from 2^31 on; every real offset is below 2^31).
    auto chunk_offset = [&](int c) {
        return active ? uint32_t((c / 9) * row_bytes + wave * 144 + 16 * (c % 9)) : 0x80000000u;
    };
    const uint32_t vo0 = chunk_offset(lane);
    const uint32_t vo1 = chunk_offset(64 + lane);
    const uint32_t vo2 = chunk_offset(128 + (lane >> 2)) + 4 * (lane & 3);
    auto issue = [&](auto b, int k) {
        uint8_t* dst = slot(b) + wave * kItemBytes;
        const uint32_t base = uint32_t((w0 + k * G) * TB);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)dst, 16, base + vo0, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(dst + 1024), 16, base + vo1, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(dst + 2048), 4, base + vo2, 0, 0, 0);
    };
    // Every wave requests its x before any wave requests weights: a CU returns loads in
    // order, and x queued behind the weight stream would arrive microseconds late.
    // Only the first item is requested before the x staging: items queued ahead of it hold
    // up the staging barrier (the CU accepts loads in order), so the rest follow it.
    asm volatile("s_barrier" ::: "memory");
    issue(std::integral_constant<int, 0>{}, 0);

    // Stage x: 8 lanes per 32-block, 4 values (one float4) per lane; plane-major digits.
    if (tid < nquads) {   // uniform per wave: K is a multiple of 256
        const float4 v = xe;
        float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        a = lanes8_max(a);
        // amax = m * 2^E, m in [0.5, 1): scale by 2^(21 - E) puts the block in [2^20, 2^21)
        const int k = kFracBits - __builtin_amdgcn_frexp_expf(a);
        uint32_t d0, d1, d2;
        transpose3(digits3(v.x, k), digits3(v.y, k), digits3(v.z, k), digits3(v.w, k), d0, d1, d2);
        *reinterpret_cast<uint32_t*>(xp + 4 * tid) = d0;
        *reinterpret_cast<uint32_t*>(xp + K + 4 * tid) = d1;
        *reinterpret_cast<uint32_t*>(xp + 2 * K + 4 * tid) = d2;
        float sm = (v.x + v.y) + (v.z + v.w);
        sm = lanes8_sum(sm);
        if ((tid & 7) == 0) {
            sums[tid >> 3] = sm;
            ex[tid >> 3] = -k;
        }
    }
    wait_barrier<3>();   // x staged; the first item's loads stay in flight
    static_for<NB - 2>([&](auto b) {
        constexpr int B = decltype(b)::value + 1;
        issue(std::integral_constant<int, B>{}, B);
    });

    // Lane roles: B column n (row n of the tile) with unit q of this wave's super-block;
    // A row n of lane group q is digit plane n & 3 of unit q's values when n / 4 == q and
    // n & 3 < 3, else zero.
    const int n = lane & 15, q = lane >> 4;
    const int sb = active ? wave : 0;
    v4i a0 = {0, 0, 0, 0}, a1 = a0, a2 = a0, a3 = a0;
    if ((n >> 2) == q && (n & 3) < 3) {
        const int8_t* ap = xp + (n & 3) * K + 256 * sb + 64 * q;
        a0 = *reinterpret_cast<const v4i*>(ap);
        a1 = *reinterpret_cast<const v4i*>(ap + 16);
        a2 = *reinterpret_cast<const v4i*>(ap + 32);
        a3 = *reinterpret_cast<const v4i*>(ap + 48);
    }
    const int2 e2 = *reinterpret_cast<const int2*>(ex + 8 * sb + 2 * q);        // sub-blocks 2q, 2q + 1
    const float2 s2 = *reinterpret_cast<const float2*>(sums + 8 * sb + 2 * q);
    // (scale, min) bytes of sub-blocks 2q, 2q + 1 from the packed 12-byte field (per-lane q)
    const uint32_t sc_shift = 16u * uint32_t(q & 1);
    wait_barrier<(NB - 1) * 3>();   // x no longer read: its LDS now takes the partials

    auto compute = [&](const uint8_t* it, int k) {
        const uint8_t* blk = it + n * 144;
        const uint4 hd = *reinterpret_cast<const uint4*>(blk);
        const v4i c0 = *reinterpret_cast<const v4i*>(blk + 16 + 32 * q);
        const v4i c1 = *reinterpret_cast<const v4i*>(blk + 32 + 32 * q);
        const v4i z = {0, 0, 0, 0};
        v4i clo = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, c0 & 0x0F0F0F0F, z, 0, 0, 0);
        clo = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, c1 & 0x0F0F0F0F, clo, 0, 0, 0);
        v4i chi = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, (c0 >> 4) & 0x0F0F0F0F, z, 0, 0, 0);
        chi = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, (c1 >> 4) & 0x0F0F0F0F, chi, 0, 0, 0);
        const int ilo = combine3(clo), ihi = combine3(chi);
        const uint32_t t0 = hd.y >> sc_shift, t1 = hd.z >> sc_shift, t2 = hd.w >> sc_shift;
        const uint32_t sc_hi = (t2 & 0x0F0Fu) | ((t0 >> 2) & 0x3030u);
        const uint32_t mn_hi = ((t2 >> 4) & 0x0F0Fu) | ((t1 >> 2) & 0x3030u);
        const uint32_t scp = q >= 2 ? sc_hi : (t0 & 0x3F3Fu);
        const uint32_t mnp = q >= 2 ? mn_hi : (t1 & 0x3F3Fu);
        const float d = half_bits_to_float(hd.x & 0xFFFFu);
        const float dmin = half_bits_to_float(hd.x >> 16);
        const float codes = ldexpf(ubyte_f<0>(scp) * float(ilo), e2.x) + ldexpf(ubyte_f<1>(scp) * float(ihi), e2.y);
        const float mins = fmaf(ubyte_f<0>(mnp), s2.x, ubyte_f<1>(mnp) * s2.y);
        const float r = sum_lane_groups(fmaf(d, codes, -dmin * mins));
        if (q == 0) part[(k * kTileRows + n) * kWaves + wave] = r;
    };

    // Item k sits in slot k % NB.  Whole ring periods, then the tail: with no condition
    // inside the loop the compiler counts the loads in flight exactly.
    constexpr int kInFlight = (NB - 1) * 3;   // loads of the NB - 1 items after item k
    static_assert(kInFlight < 16, "vmcnt immediate");
    auto step = [&](auto b, int k) {
        constexpr int B = decltype(b)::value;
        issue(std::integral_constant<int, (B + NB - 1) % NB>{}, k + NB - 1);   // the slot of item k - 1
        __builtin_amdgcn_s_waitcnt(kInFlight | 0x0F70);                       // item k has landed
        compute(slot(b) + wave * kItemBytes, k);
    };
    if (active) {
        int k0 = 0;
        for (; k0 + NB <= tiles; k0 += NB) static_for<NB>([&](auto b) { step(b, k0 + decltype(b)::value); });
        static_for<NB>([&](auto b) {
            if (k0 + decltype(b)::value < tiles) step(b, k0 + decltype(b)::value);
        });
    }
    wait_barrier<0>();   // every partial written (and the loads past the end have landed)

    // Row sums: lane j of the four lanes of row r adds the partials of waves 4j .. 4j + 3
    // (one 16-byte LDS read; waves past the row's super-blocks wrote none and count zero).
    // tiles * 16 rows * 4 lanes <= kThreads (kMaxTilesPerGroup).
    const int wl = SB < kWaves ? SB : kWaves;
    const int r = tid >> 2, j = tid & 3;
    float s = 0.f;
    if (r < tiles * kTileRows) {
        const float4 v = *reinterpret_cast<const float4*>(part + r * kWaves + 4 * j);
        s = ((4 * j < wl ? v.x : 0.f) + (4 * j + 1 < wl ? v.y : 0.f)) +
            ((4 * j + 2 < wl ? v.z : 0.f) + (4 * j + 3 < wl ? v.w : 0.f));
    }
    s = lanes8_sum<2>(s);
    if (j == 0 && r < tiles * kTileRows) {
        const int row = (w0 + (r / kTileRows) * G) * kTileRows + r % kTileRows;
        if (row < N) y[row] = s;
    }
}


// ------------------------------------------------------------------ long rows
// More than 16 super-blocks per row (e.g. the 7B ffn_down 3584 x 18944, 74 super-blocks)
// and at most 16 rows per CU: each workgroup owns one tile of TR <= 16 consecutive rows,
// TR = ceil(N / G), so that the G workgroups split N evenly, and its 16 waves share the
// tile's super-blocks: wave w takes super-blocks w, w + 16, w + 32, ...  (At any moment
// the GPU then reads 16 consecutive super-blocks, 2304 contiguous bytes, of every row.)
// An item is one super-block of the tile's rows (TR x 144 bytes; the lanes of rows past
// TR read past the end of the buffer: zeros, no traffic), streamed into the wave's LDS
// ring as in the kernel above, together with that super-block's 256 x values (one float4
// per lane, into registers).  When the item has landed the wave turns its x into the
// exact digit form of the kernel above in its own 832 bytes of LDS (no workgroup
// barrier: a wave reads back only what it wrote, and one wave's LDS operations complete
// in order), then runs the same four MFMAs.  A lane accumulates its unit's share of its
// row over the wave's items, in item order; the four lanes of a row, then the 16 waves,
// are summed at the end in a fixed order (deterministic).  One item in flight per wave
// (a ring of two slots): rings of three and four slots measured slower (more rows'
// fragments in flight at once), and so did staggering the item order across CUs.
constexpr int kLongRing = 2;
constexpr uint32_t kPastEnd = 0x7FFF0000u;   // a buffer offset past the end of any matrix this kernel takes

//
// On Q4_K's row-tiled layout (TILED) the tile is a group of that layout, TR its rows, and an
// item is one contiguous run of TR x 144 bytes; the kernel is otherwise the same, and so are
// its results, bit for bit.
template <int NB, bool TILED>
__global__ __launch_bounds__(kThreads) void gemv_mfma_q4k_long_kernel(const uint8_t* __restrict__ W,
                                                                       const float* __restrict__ x,
                                                                       float* __restrict__ y, int N, int K,
                                                                       int row_bytes, int TR, int nbytes) {
    __shared__ __attribute__((aligned(16))) uint8_t ring0[kWaves * kItemBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[kWaves * kItemBytes];
    __shared__ __attribute__((aligned(16))) uint8_t ring2[NB > 2 ? kWaves * kItemBytes : 16];
    __shared__ __attribute__((aligned(16))) uint8_t ring3[NB > 3 ? kWaves * kItemBytes : 16];
    __shared__ __attribute__((aligned(16))) int8_t xs[kWaves * 768];   // per wave: 3 digit planes of 256 values
    __shared__ __attribute__((aligned(16))) int xex[kWaves * 8];       // per wave: 8 block exponents
    __shared__ __attribute__((aligned(16))) float xsum[kWaves * 8];    // per wave: 8 block sums
    __shared__ __attribute__((aligned(16))) float part[kTileRows * kWaves];
    auto slot = [&](auto b) -> uint8_t* {
        constexpr int B = decltype(b)::value;
        if constexpr (B == 0) return ring0;
        else if constexpr (B == 1) return ring1;
        else if constexpr (B == 2) return ring2;
        else return ring3;
    };

    const int SB = K >> 8;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r0 = blockIdx.x * TR;
    const int rows = min(TR, N - r0);
    const int items = (SB - wave + kWaves - 1) / kWaves;   // super-blocks wave, wave + 16, ... (>= 1: SB > 16)

    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W), 0, nbytes, kBufferWord3);
    // byte offset of 16-byte chunk c (row c / 9, chunk c % 9 of its block) within an item
    auto chunk_offset = [&](int c) {
        return TILED ? uint32_t(16 * c) : uint32_t((c / 9) * row_bytes + 16 * (c % 9));
    };
    const int c0 = lane, c1 = 64 + lane, c2 = 128 + (lane >> 2);
    const bool live0 = c0 / 9 < rows, live1 = c1 / 9 < rows, live2 = c2 / 9 < rows;
    const uint32_t vo0 = chunk_offset(c0), vo1 = chunk_offset(c1), vo2 = chunk_offset(c2) + 4 * (lane & 3);
    const uint32_t tile0 = uint32_t(r0) * uint32_t(row_bytes);
    float4 xr[NB];
    // Item i: x of super-block wave + 16 i (a float4 per lane, into registers), then the
    // super-block's TR rows (into the slot).  Items past the wave's last read x of its
    // last super-block and move no weight bytes.
    auto issue = [&](auto b, int i) {
        constexpr int B = decltype(b)::value;
        uint8_t* dst = slot(b) + wave * kItemBytes;
        const bool in = i < items;
        const int sb = wave + kWaves * (in ? i : items - 1);
        xr[B] = reinterpret_cast<const float4*>(x + 256 * sb)[lane];
        const uint32_t base = tile0 + uint32_t(sb) * (TILED ? uint32_t(TR * 144) : 144u);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)dst, 16, in && live0 ? base + vo0 : kPastEnd, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(dst + 1024), 16, in && live1 ? base + vo1 : kPastEnd, 0,
                                                 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(dst + 2048), 4, in && live2 ? base + vo2 : kPastEnd, 0,
                                                 0, 0);
    };
    static_for<NB - 1>([&](auto b) { issue(b, decltype(b)::value); });
    // Every wave's first item is requested before any wave requests its second: a CU serves
    // loads roughly in issue order, and without this the last waves to start found the
    // first two items of every other wave ahead of their first (ffn_down 3584 x 18944:
    // 11.0 -> 10.8 us).  No wait for memory (a plain s_barrier, not __syncthreads).
    asm volatile("s_barrier" ::: "memory");

    const int n = lane & 15, q = lane >> 4;
    const bool a_lane = (n >> 2) == q && (n & 3) < 3;
    const uint32_t sc_shift = 16u * uint32_t(q & 1);
    int8_t* my_xs = xs + wave * 768;
    int* my_ex = xex + wave * 8;
    float* my_sum = xsum + wave * 8;
    float acc = 0.f;

    auto compute = [&](const uint8_t* it, const float4 v) {
        // Stage this super-block's x: lane l holds values 4l .. 4l + 3, 8 lanes per 32-block.
        float a = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        a = lanes8_max(a);
        const int k = kFracBits - __builtin_amdgcn_frexp_expf(a);
        uint32_t d0, d1, d2;
        transpose3(digits3(v.x, k), digits3(v.y, k), digits3(v.z, k), digits3(v.w, k), d0, d1, d2);
        *reinterpret_cast<uint32_t*>(my_xs + 4 * lane) = d0;
        *reinterpret_cast<uint32_t*>(my_xs + 256 + 4 * lane) = d1;
        *reinterpret_cast<uint32_t*>(my_xs + 512 + 4 * lane) = d2;
        float sm = (v.x + v.y) + (v.z + v.w);
        sm = lanes8_sum(sm);
        if ((lane & 7) == 0) {
            my_sum[lane >> 3] = sm;
            my_ex[lane >> 3] = -k;
        }
        // (LDS operations of one wave complete in order: the reads below see the writes.)
        v4i a0 = {0, 0, 0, 0}, a1 = a0, a2 = a0, a3 = a0;
        if (a_lane) {
            const int8_t* ap = my_xs + (n & 3) * 256 + 64 * q;
            a0 = *reinterpret_cast<const v4i*>(ap);
            a1 = *reinterpret_cast<const v4i*>(ap + 16);
            a2 = *reinterpret_cast<const v4i*>(ap + 32);
            a3 = *reinterpret_cast<const v4i*>(ap + 48);
        }
        const int2 e2 = *reinterpret_cast<const int2*>(my_ex + 2 * q);
        const float2 s2 = *reinterpret_cast<const float2*>(my_sum + 2 * q);
        const uint8_t* blk = it + n * 144;
        const uint4 hd = *reinterpret_cast<const uint4*>(blk);
        const v4i c0w = *reinterpret_cast<const v4i*>(blk + 16 + 32 * q);
        const v4i c1w = *reinterpret_cast<const v4i*>(blk + 32 + 32 * q);
        const v4i z = {0, 0, 0, 0};
        v4i clo = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, c0w & 0x0F0F0F0F, z, 0, 0, 0);
        clo = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, c1w & 0x0F0F0F0F, clo, 0, 0, 0);
        v4i chi = __builtin_amdgcn_mfma_i32_16x16x64_i8(a2, (c0w >> 4) & 0x0F0F0F0F, z, 0, 0, 0);
        chi = __builtin_amdgcn_mfma_i32_16x16x64_i8(a3, (c1w >> 4) & 0x0F0F0F0F, chi, 0, 0, 0);
        const int ilo = combine3(clo), ihi = combine3(chi);
        const uint32_t t0 = hd.y >> sc_shift, t1 = hd.z >> sc_shift, t2 = hd.w >> sc_shift;
        const uint32_t sc_hi = (t2 & 0x0F0Fu) | ((t0 >> 2) & 0x3030u);
        const uint32_t mn_hi = ((t2 >> 4) & 0x0F0Fu) | ((t1 >> 2) & 0x3030u);
        const uint32_t scp = q >= 2 ? sc_hi : (t0 & 0x3F3Fu);
        const uint32_t mnp = q >= 2 ? mn_hi : (t1 & 0x3F3Fu);
        const float d = half_bits_to_float(hd.x & 0xFFFFu);
        const float dmin = half_bits_to_float(hd.x >> 16);
        const float codes = ldexpf(ubyte_f<0>(scp) * float(ilo), e2.x) + ldexpf(ubyte_f<1>(scp) * float(ihi), e2.y);
        const float mins = fmaf(ubyte_f<0>(mnp), s2.x, ubyte_f<1>(mnp) * s2.y);
        acc += fmaf(d, codes, -dmin * mins);
    };

    constexpr int kInFlight = (NB - 1) * 4;   // x and weight loads of the NB - 1 items after item i
    static_assert(kInFlight < 16, "vmcnt immediate");
    auto step = [&](auto b, int i) {
        constexpr int B = decltype(b)::value;
        issue(std::integral_constant<int, (B + NB - 1) % NB>{}, i + NB - 1);   // the slot of item i - 1
        __builtin_amdgcn_s_waitcnt(kInFlight | 0x0F70);                       // item i has landed
        compute(slot(b) + wave * kItemBytes, xr[B]);
    };
    int i0 = 0;
    for (; i0 + NB <= items; i0 += NB) static_for<NB>([&](auto b) { step(b, i0 + decltype(b)::value); });
    static_for<NB>([&](auto b) {
        if (i0 + decltype(b)::value < items) step(b, i0 + decltype(b)::value);
    });

    const float r = sum_lane_groups(acc);
    if (q == 0) part[n * kWaves + wave] = r;
    wait_barrier<0>();   // every partial written (and the loads past the end have landed)

    const int rr = tid >> 2, j = tid & 3;
    float sum = 0.f;
    if (rr < kTileRows) {
        const float4 v = *reinterpret_cast<const float4*>(part + rr * kWaves + 4 * j);
        sum = (v.x + v.y) + (v.z + v.w);
    }
    sum = lanes8_sum<2>(sum);
    if (j == 0 && rr < rows) y[r0 + rr] = sum;
}


// ------------------------------------------------------------------ whole tiles
// Q6_K blocks are 210 bytes: neither the blocks nor the rows sit on 16-byte boundaries,
// but a tile of 16 consecutive rows is 16 x row_bytes, a whole number of 16-byte chunks.
// So the workgroup streams whole tiles: lane i reads chunks i, i + 1024, ... of the tile
// into registers (16-byte loads, consecutive lanes on consecutive bytes), D tiles ahead,
// and writes them to one of two LDS slots, so a tile is one contiguous copy of its bytes
// in LDS.  A workgroup barrier per tile separates the slot being written from the one
// being read.  Tiles are dealt round-robin as above (tile t to workgroup t % G).
//
// Wave w computes super-block w of the tile's 16 rows with four v_mfma_i32_16x16x64_i8,
// one per quarter t of the super-block's 16 runs of 16 values: lane group q takes run
// g = 4t + q, A row 4q + p holds digit plane p of the run's x values and B column n the
// run's 16 codes of row n (16 consecutive ql bytes, one nibble, and 16 consecutive qh
// bytes, two bits).  So lane (n, q) receives the exact sums over run g of code * v per
// plane, and applies the run's signed sub-scale and the code offset 32 through the run's
// f32 sum of x:
//   y[n] += d * sum_t sc[4t + q] * (2^e * sum(code * v) - 32 * sum(x)).
// Blocks start at even byte offsets in LDS; each 16-byte field is read as the five
// aligned dwords that cover it and realigned with v_alignbyte.
//
// The kernel takes any block type through TiledItem (bytes per 256 values and the lane's
// share of a super-chunk; the per-wave kernel further down uses the Q8_0, Q4_0 and Q5_0 items).
// Q8_0, Q4_0, Q4_1, Q5_0, Q5_1 and Q5_K run through this whole-tile stream passed the
// parity tests but measured slower than the vector kernel on the 7B ffn_up shape (their
// decode is light, and the per-tile barrier and realignment cost more than they save), so
// only Q6_K is routed here.
constexpr uint32_t kTiledPastEnd = 0x80000000u;   // a buffer offset past the end of any matrix this kernel takes

// 16 bytes at an even LDS address: the five aligned dwords that cover them, realigned
__device__ __forceinline__ uint4 lds_seg16(const uint8_t* p) {
    const uint32_t a = uint32_t(reinterpret_cast<uintptr_t>(p));
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p - (a & 3));
    const uint32_t sh = a & 3;
    const uint32_t w0 = q[0], w1 = q[1], w2 = q[2], w3 = q[3], w4 = q[4];
    return make_uint4(__builtin_amdgcn_alignbyte(w1, w0, sh), __builtin_amdgcn_alignbyte(w2, w1, sh),
                      __builtin_amdgcn_alignbyte(w3, w2, sh), __builtin_amdgcn_alignbyte(w4, w3, sh));
}
// The same when p is known to be 4-byte aligned: four dword reads, nothing to realign.
template <bool ALIGNED>
__device__ __forceinline__ uint4 lds_seg16_if(const uint8_t* p) {
    if constexpr (ALIGNED) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
        return make_uint4(q[0], q[1], q[2], q[3]);
    } else {
        return lds_seg16(p);
    }
}
__device__ __forceinline__ float lds_f16(const uint8_t* p) {
    return half_bits_to_float(uint32_t(*reinterpret_cast<const uint16_t*>(p)));
}
__device__ __forceinline__ v4i as_v4i(uint4 v) { return v4i{int(v.x), int(v.y), int(v.z), int(v.w)}; }
// the low (hi = 0) or high (hi = 1) nibbles of 16 bytes, one per byte
__device__ __forceinline__ uint4 nib4(uint4 v, int hi) {
    const int s = 4 * hi;
    return make_uint4((v.x >> s) & 0x0F0F0F0Fu, (v.y >> s) & 0x0F0F0F0Fu, (v.z >> s) & 0x0F0F0F0Fu,
                      (v.w >> s) & 0x0F0F0F0Fu);
}
// signed byte k (0..3) of a dword
__device__ __forceinline__ float sbyte_f(uint32_t v, int k) { return float(int32_t(v << (24 - 8 * k)) >> 24); }


// Per type: bytes per 256 values, and the lane's share of one super-chunk of its row.
// row: the row's bytes in LDS; sc: super-chunk index; q: lane group; a, e, sx: the
// lane's x digits, exponents and f32 x sums for runs 4t + q.
template <int QT> struct TiledItem;

template <> struct TiledItem<kQ6_K> {
    static constexpr int kSBBytes = 210;
    __device__ static float run(const uint8_t* row, int sc, int q, const v4i (&a)[4], const int (&e)[4],
                                const float (&sx)[4]) {
        const uint8_t* blk = row + sc * kSBBytes;
        const uint4 scw = lds_seg16(blk + 192);
        const uint32_t sc4[4] = {scw.x, scw.y, scw.z, scw.w};
        const uint32_t s_lo = 2u * uint32_t(q >> 1);   // qh bit pair of the low-nibble runs (t even)
        float acc = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            // runs 8h + q (low nibbles) and 8h + 4 + q (high nibbles) share 16 ql and 16 qh bytes
            const uint4 ql = lds_seg16(blk + 64 * h + 16 * q);
            const uint4 qh = lds_seg16(blk + 128 + 32 * h + 16 * (q & 1));
            const uint32_t L[4] = {ql.x, ql.y, ql.z, ql.w}, H[4] = {qh.x, qh.y, qh.z, qh.w};
            v4i clo, chi;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                clo[i] = int((L[i] & 0x0F0F0F0Fu) | (((H[i] >> s_lo) & 0x03030303u) << 4));
                chi[i] = int(((L[i] >> 4) & 0x0F0F0F0Fu) | (((H[i] >> (s_lo + 4)) & 0x03030303u) << 4));
            }
            const v4i z = {0, 0, 0, 0};
            const v4i rlo = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[2 * h], clo, z, 0, 0, 0);
            const v4i rhi = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[2 * h + 1], chi, z, 0, 0, 0);
            acc = fmaf(sbyte_f(sc4[2 * h], q), fmaf(-32.0f, sx[2 * h], ldexpf(float(combine3(rlo)), e[2 * h])), acc);
            acc = fmaf(sbyte_f(sc4[2 * h + 1], q),
                       fmaf(-32.0f, sx[2 * h + 1], ldexpf(float(combine3(rhi)), e[2 * h + 1])), acc);
        }
        return lds_f16(blk + 208) * acc;
    }
};

template <> struct TiledItem<kQ8_0> {
    static constexpr int kSBBytes = 8 * 34;
    __device__ static float run(const uint8_t* row, int sc, int q, const v4i (&a)[4], const int (&e)[4],
                                const float (&)[4]) {
        float acc = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint8_t* blk = row + (8 * sc + 2 * t + (q >> 1)) * 34;   // block of run 4t + q
            const v4i c = as_v4i(lds_seg16(blk + 2 + 16 * (q & 1)));
            const v4i r = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], c, v4i{0, 0, 0, 0}, 0, 0, 0);
            acc = fmaf(lds_f16(blk), ldexpf(combine3f(r), e[t]), acc);
        }
        return acc;
    }
};

// Q4_0: run 4t + q is half h = q % 2 of block 2t + q / 2 of the super-chunk, whose values
// 16h + i take the low (h = 0) or high (h = 1) nibble of qs[i]; the code offset 8 goes
// through the run's x sum.
template <> struct TiledItem<kQ4_0> {
    static constexpr int kSBBytes = 8 * 18;
    __device__ static float run(const uint8_t* row, int sc, int q, const v4i (&a)[4], const int (&e)[4],
                                const float (&sx)[4]) {
        const int h = q & 1;
        float acc = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint8_t* blk = row + (8 * sc + 2 * t + (q >> 1)) * 18;
            const v4i c = as_v4i(nib4(lds_seg16(blk + 2), h));
            const v4i r = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], c, v4i{0, 0, 0, 0}, 0, 0, 0);
            acc = fmaf(lds_f16(blk), fmaf(-8.0f, sx[t], ldexpf(float(combine3(r)), e[t])), acc);
        }
        return acc;
    }
};

// Q5_0 (22-byte blocks: f16 d, 4 bytes of high bits, 16 bytes of nibbles): values 16h + i
// take nibble h of byte i and bit 16h + i of the high-bit word as their fifth bit, and the
// value is d * (code - 16).  Blocks start at even LDS offsets, so the high-bit word is read
// as the two aligned dwords around it.
__device__ __forceinline__ uint32_t lds_u32_a2(const uint8_t* p) {
    const uint32_t a = uint32_t(reinterpret_cast<uintptr_t>(p));
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p - (a & 3));
    return __builtin_amdgcn_alignbyte(q[1], q[0], a & 3);
}
// bits 0..3 of v to bit 0 of bytes 0..3
__device__ __forceinline__ uint32_t bits_to_bytes4(uint32_t v) { return (v * 0x00204081u) & 0x01010101u; }
template <> struct TiledItem<kQ5_0> {
    static constexpr int kSBBytes = 8 * 22;
    __device__ static float run(const uint8_t* row, int sc, int q, const v4i (&a)[4], const int (&e)[4],
                                const float (&sx)[4]) {
        const int h = q & 1;
        float acc = 0.f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint8_t* blk = row + (8 * sc + 2 * t + (q >> 1)) * 22;
            uint4 c = nib4(lds_seg16(blk + 6), h);
            const uint32_t bits = lds_u32_a2(blk + 2) >> (16 * h);
            c.x |= bits_to_bytes4(bits & 15u) << 4;
            c.y |= bits_to_bytes4((bits >> 4) & 15u) << 4;
            c.z |= bits_to_bytes4((bits >> 8) & 15u) << 4;
            c.w |= bits_to_bytes4((bits >> 12) & 15u) << 4;
            const v4i r = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[t], as_v4i(c), v4i{0, 0, 0, 0}, 0, 0, 0);
            acc = fmaf(lds_f16(blk), fmaf(-16.0f, sx[t], ldexpf(float(combine3(r)), e[t])), acc);
        }
        return acc;
    }
};

template <int QT>
constexpr int tiled_slot_bytes() { return kTileRows * kMaxSB * TiledItem<QT>::kSBBytes; }

// D: tiles in flight (register ring; two measured faster than three or four); CPL: 16-byte
// chunks per lane and tile.  The loop is unrolled over lcm(D, 2) tiles so that every ring
// and slot index is a compile-time constant.
template <int QT, int D, int CPL>
__global__ __launch_bounds__(kThreads) void gemv_tiled_kernel(const uint8_t* __restrict__ W,
                                                              const float* __restrict__ x,
                                                              float* __restrict__ y, int N, int K,
                                                              int row_bytes) {
    using Item = TiledItem<QT>;
    constexpr int kSlot = tiled_slot_bytes<QT>();
    // (16 bytes past a full slot: the aligned dwords read around a row's last block may
    // reach 2 bytes past its end)
    __shared__ __attribute__((aligned(16))) uint8_t slot0[kSlot + 16];
    __shared__ __attribute__((aligned(16))) uint8_t slot1[kSlot + 16];
    __shared__ __attribute__((aligned(16))) int8_t xp[3 * 256 * kMaxSB];   // digit planes [3][K]
    __shared__ __attribute__((aligned(16))) int ex[8 * kMaxSB];             // per 32-block
    __shared__ __attribute__((aligned(16))) float sums[16 * kMaxSB];        // per 16-run
    __shared__ __attribute__((aligned(16))) float part[2][kTileRows * kWaves];
    auto slot = [&](auto b) -> uint8_t* {
        if constexpr (decltype(b)::value == 0) return slot0;
        else return slot1;
    };

    const int SB = K >> 8;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x, w0 = blockIdx.x;
    const int T = (N + kTileRows - 1) / kTileRows;
    const int tiles = (T - w0 + G - 1) / G;   // this workgroup's: global tiles w0 + k G
    const uint32_t TB = uint32_t(kTileRows) * uint32_t(row_bytes);
    const int chunks = row_bytes;             // 16-byte chunks per tile: 16 x row_bytes / 16

    const int nquads = K >> 2;
    float4 xe = {};
    if (tid < nquads) xe = reinterpret_cast<const float4*>(x)[tid];

    // The matrix as one buffer: rows past the last read as zeros.
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W), 0, N * row_bytes, kBufferWord3);
    uint4 R[D][CPL];
    auto issue = [&](auto r, int k) {
        constexpr int J = decltype(r)::value;
        const uint32_t base = k < tiles ? uint32_t(w0 + k * G) * TB : kTiledPastEnd;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = tid + j * kThreads;
            const uint32_t off = c < chunks ? base + 16u * uint32_t(c) : kTiledPastEnd;
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
            R[J][j] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    };
    auto store = [&](auto r, auto b) {
        constexpr int J = decltype(r)::value;
        uint8_t* dst = slot(b);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = tid + j * kThreads;
            // CPL = ceil(chunks / 1024): only the last round of chunks is partial
            if (j < CPL - 1 || c < chunks) *reinterpret_cast<uint4*>(dst + 16 * c) = R[J][j];
        }
    };
    asm volatile("s_barrier" ::: "memory");   // every wave's x requested before any weights
    static_for<D>([&](auto r) { issue(r, decltype(r)::value); });

    // Stage x: digit planes and a 21-bit exponent per 32-block, as above, and the f32 sum
    // of every 16-value run (four lanes).
    if (tid < nquads) {   // uniform per wave: K is a multiple of 256
        const float4 v = xe;
        float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        am = lanes8_max(am);
        const int k = kFracBits - __builtin_amdgcn_frexp_expf(am);
        uint32_t d0, d1, d2;
        transpose3(digits3(v.x, k), digits3(v.y, k), digits3(v.z, k), digits3(v.w, k), d0, d1, d2);
        *reinterpret_cast<uint32_t*>(xp + 4 * tid) = d0;
        *reinterpret_cast<uint32_t*>(xp + K + 4 * tid) = d1;
        *reinterpret_cast<uint32_t*>(xp + 2 * K + 4 * tid) = d2;
        float sm = (v.x + v.y) + (v.z + v.w);
        sm = lanes8_sum<2>(sm);
        if ((tid & 3) == 0) sums[tid >> 2] = sm;
        if ((tid & 7) == 0) ex[tid >> 3] = -k;
    }
    __syncthreads();

    // Lane roles as in the Q4_K kernel: column n = row n of the tile, lane group q = run
    // 4t + q of this wave's super-chunk in MFMA t.
    const bool active = wave < SB;   // uniform
    const int sc = active ? wave : 0;
    const int n = lane & 15, q = lane >> 4;
    v4i a[4];
    int e[4];
    float sx[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        a[t] = v4i{0, 0, 0, 0};
        if ((n >> 2) == q && (n & 3) < 3)
            a[t] = *reinterpret_cast<const v4i*>(xp + (n & 3) * K + 256 * sc + 64 * t + 16 * q);
        e[t] = ex[8 * sc + 2 * t + (q >> 1)];
        sx[t] = sums[16 * sc + 4 * t + q];
    }

    auto compute = [&](const uint8_t* tile, float* pt) {
        const float r = sum_lane_groups(Item::run(tile + n * row_bytes, sc, q, a, e, sx));
        if (q == 0) pt[n * kWaves + wave] = r;
    };
    // Row sums of a tile's partials (wave kWaves - 1, idle in compute when SB < 16):
    // lane j of row r's four lanes adds waves 4j .. 4j + 3, then two lane swaps.
    auto row_sums = [&](const float* pt, int k) {
        if (wave != kWaves - 1) return;
        const int r = lane >> 2, j = lane & 3;
        const float4 v = *reinterpret_cast<const float4*>(pt + r * kWaves + 4 * j);
        float s = ((4 * j < SB ? v.x : 0.f) + (4 * j + 1 < SB ? v.y : 0.f)) +
                  ((4 * j + 2 < SB ? v.z : 0.f) + (4 * j + 3 < SB ? v.w : 0.f));
        s = lanes8_sum<2>(s);
        const int row = (w0 + k * G) * kTileRows + r;
        if (j == 0 && row < N) y[row] = s;
    };

    // Tile 0 into slot 0; then per tile k: compute it, sum the rows of tile k - 1, move
    // tile k + 1 from its registers into the other slot and refill those registers with
    // tile k + 1 + D, barrier.
    if (tiles > 0) {
        store(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
        issue(std::integral_constant<int, 0>{}, D);
    }
    __syncthreads();
    constexpr int P = D % 2 == 0 ? D : 2 * D;   // lcm(D, 2)
    auto body = [&](auto i_c, int k) {
        constexpr int I = decltype(i_c)::value;   // k % P
        if (active) compute(slot(std::integral_constant<int, I % 2>{}), part[I % 2]);
        if (k > 0) row_sums(part[(I + 1) % 2], k - 1);
        if (k + 1 < tiles) {
            store(std::integral_constant<int, (I + 1) % D>{}, std::integral_constant<int, (I + 1) % 2>{});
            issue(std::integral_constant<int, (I + 1) % D>{}, k + 1 + D);
        }
        __syncthreads();
    };
    int k0 = 0;
    for (; k0 + P <= tiles; k0 += P) static_for<P>([&](auto i) { body(i, k0 + decltype(i)::value); });
    static_for<P>([&](auto i) {
        if (k0 + decltype(i)::value < tiles) body(i, k0 + decltype(i)::value);
    });
    if (tiles > 0) row_sums(part[(tiles - 1) % 2], tiles - 1);
}


// ------------------------------------------------------------------ Q6_K, a few q8 rows
// The product of mq_gemm for M <= 8 activation rows already quantized to q8 blocks, on the
// whole-tile stream above: the weight bytes are read once for all rows.  A is now the
// rows' int8 codes themselves: lane (i, q) holds, for i / 4 == q, the 16 codes of run
// 4t + q of activation row i % 4 (+ 4 in the second MFMA of a quarter, for M > 4), so
// lane (n, q) receives the exact int32 dots of that run with weight row n for four
// activation rows.  Each result is the run's block dot sum((c - 32) q) directly: for
// four rows a first MFMA of the same A with B = -32 in every byte seeds the accumulator
// with -32 sum(q); for eight rows (whose registers are short) B holds the codes minus 32
// as signed bytes instead.  And
//   Y[m][n] = sum over runs of d * sc_g * dx[m][block] * dot.
// Row m's arithmetic does not depend on the other rows or on M: the product of M <= 8
// rows equals, row by row, the product of each row alone, bit for bit.
// Tiles ahead in registers: one, as for the f32 kernel above (two measured 5% slower on the
// vocab head at M = 8).
constexpr int kQ8TiledDepth = 1;
template <int MR, bool DUMP, int CPL>
__global__ __launch_bounds__(kThreads) void gemv_q8_q6k_kernel(const uint8_t* __restrict__ W,
                                                               const int8_t* __restrict__ codes,
                                                               const float* __restrict__ xscale,
                                                               float* __restrict__ Y, int32_t* __restrict__ dots,
                                                               int M, int N, int K, int row_bytes) {
    constexpr int kSlot = tiled_slot_bytes<kQ6_K>();
    constexpr int H = MR / 4;   // MFMAs per quarter
    constexpr int kStage = MR * 256 * kMaxSB;
    static_assert(MR == 4 || MR == 8, "row groups of four");
    __shared__ __attribute__((aligned(16))) uint8_t slot0[kSlot + 16];
    __shared__ __attribute__((aligned(16))) uint8_t slot1[kSlot + 16];
    __shared__ __attribute__((aligned(16))) uint8_t stage[kStage];                       // codes [MR][K], rows M.. zero
    __shared__ __attribute__((aligned(16))) float dxT[8 * kMaxSB][MR];                    // block scales [block][row]
    __shared__ __attribute__((aligned(16))) float part[2][MR * kTileRows * kWaves];       // [m][row][wave]
    auto slot = [&](auto b) -> uint8_t* {
        if constexpr (decltype(b)::value == 0) return slot0;
        else return slot1;
    };

    const int SB = K >> 8, KB = K >> 5;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x, w0 = blockIdx.x;
    const int T = (N + kTileRows - 1) / kTileRows;
    const int tiles = (T - w0 + G - 1) / G;
    const uint32_t TB = uint32_t(kTileRows) * uint32_t(row_bytes);
    const int chunks = row_bytes;

    // The rows' codes and block scales first (loads complete in issue order).
    constexpr int kCodeLoads = kStage / 16 / kThreads;   // 16-byte chunks per lane
    uint4 xc[kCodeLoads];
    const int rowchunks = K >> 4;
#pragma unroll
    for (int j = 0; j < kCodeLoads; ++j) {
        const int c = tid + j * kThreads, r = c / rowchunks;
        xc[j] = make_uint4(0, 0, 0, 0);
        if (r < M) xc[j] = reinterpret_cast<const uint4*>(codes)[c];   // rows are contiguous: chunk c of the plane
    }
    float dxv = 0.f;
    const int br = tid / MR, rr = tid % MR;   // dxT entry [br][rr]
    if (br < KB && rr < M) dxv = xscale[int64_t(rr) * KB + br];

    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W), 0, N * row_bytes, kBufferWord3);
    constexpr int QD = kQ8TiledDepth;   // tiles ahead in registers
    uint4 R[QD][CPL];
    auto issue = [&](auto r, int k) {
        constexpr int J = decltype(r)::value;
        const uint32_t base = k < tiles ? uint32_t(w0 + k * G) * TB : kTiledPastEnd;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = tid + j * kThreads;
            const uint32_t off = c < chunks ? base + 16u * uint32_t(c) : kTiledPastEnd;
            const auto v = __builtin_amdgcn_raw_buffer_load_b128(rw, off, 0, 0);
            R[J][j] = make_uint4(v[0], v[1], v[2], v[3]);
        }
    };
    auto store = [&](auto r, auto b) {
        constexpr int J = decltype(r)::value;
        uint8_t* dst = slot(b);
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = tid + j * kThreads;
            if (j < CPL - 1 || c < chunks) *reinterpret_cast<uint4*>(dst + 16 * c) = R[J][j];
        }
    };
    asm volatile("s_barrier" ::: "memory");   // every wave's activations requested before any weights
    issue(std::integral_constant<int, 0>{}, 0);
    if constexpr (QD == 2) issue(std::integral_constant<int, 1>{}, 1);

#pragma unroll
    for (int j = 0; j < kCodeLoads; ++j) *reinterpret_cast<uint4*>(stage + 16 * (tid + j * kThreads)) = xc[j];
    if (br < KB) dxT[br][rr] = dxv;
    __syncthreads();

    const bool active = wave < SB;   // uniform
    const int sc = active ? wave : 0;
    const int n = lane & 15, q = lane >> 4;
    // A operands (read per item: registers are short): lanes with n / 4 == q read row
    // n % 4 + 4h of the staged codes, the others hold zeros
    const bool a_lane = (n >> 2) == q;
    const uint8_t* a_src = stage + (n & 3) * K + 256 * sc + 16 * q;

    // A block starts 2-byte aligned in the tile; with an even number of super-blocks per row
    // its offset mod 4 depends on the super-block only (the wave's), so a wave whose blocks
    // start on dwords reads its segments without realigning them.
    const bool dword_blocks = ((row_bytes | (sc * TiledItem<kQ6_K>::kSBBytes)) & 3) == 0;   // uniform
    auto compute = [&](auto aligned_c, const uint8_t* tile, float* pt, int k) __attribute__((always_inline)) {
        constexpr bool AL = decltype(aligned_c)::value;
        const uint8_t* blk = tile + n * row_bytes + sc * TiledItem<kQ6_K>::kSBBytes;
        const uint4 scw = lds_seg16_if<AL>(blk + 192);
        const uint32_t sc4[4] = {scw.x, scw.y, scw.z, scw.w};
        const float d = lds_f16(blk + 208);
        const uint32_t s_lo = 2u * uint32_t(q >> 1);
        const int row = (w0 + k * G) * kTileRows + n;
        float acc[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[m] = 0.f;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            // (one half at a time: hoisting the second half's reads over the first would
            // run out of registers)
            __builtin_amdgcn_sched_barrier(0);
            const uint4 ql = lds_seg16_if<AL>(blk + 64 * hh + 16 * q);
            const uint4 qh = lds_seg16_if<AL>(blk + 128 + 32 * hh + 16 * (q & 1));
            const uint32_t L[4] = {ql.x, ql.y, ql.z, ql.w}, Hb[4] = {qh.x, qh.y, qh.z, qh.w};
#pragma unroll
            for (int part_t = 0; part_t < 2; ++part_t) {
                __builtin_amdgcn_sched_barrier(0);
                const int t = 2 * hh + part_t;   // low nibbles, then high nibbles
                v4i c;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t lo = (L[i] >> (4 * part_t)) & 0x0F0F0F0Fu;
                    const uint32_t hi = (Hb[i] >> (s_lo + 4 * part_t)) & 0x03030303u;   // the 2 high bits, per byte
                    if constexpr (MR == 4) {
                        c[i] = int(lo | (hi << 4));
                    } else {
                        // code - 32 as signed bytes: the high bits h = 0..3 of code = 16 h + lo
                        // give the byte's top nibble h - 2 (0xE, 0xF, 0x0, 0x1), looked up per
                        // byte with v_perm_b32 (selector bytes 0..3 pick bytes of 0x1000F0E0)
                        c[i] = int(__builtin_amdgcn_perm(0u, 0x1000F0E0u, hi) | lo);
                    }
                }
                const float f = d * sbyte_f(sc4[t], q);
                const float* dxb = dxT[8 * sc + 2 * t + (q >> 1)];
#pragma unroll
                for (int h = 0; h < H; ++h) {
                    v4i av = {0, 0, 0, 0};
                    if (a_lane) av = *reinterpret_cast<const v4i*>(a_src + 4 * h * K + 64 * t);
                    v4i off = {0, 0, 0, 0};
                    if constexpr (MR == 4) {
                        const v4i m32 = {int(0xE0E0E0E0u), int(0xE0E0E0E0u), int(0xE0E0E0E0u), int(0xE0E0E0E0u)};
                        off = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, m32, off, 0, 0, 0);
                    }
                    const v4i C = __builtin_amdgcn_mfma_i32_16x16x64_i8(av, c, off, 0, 0, 0);
                    const float4 dx4 = *reinterpret_cast<const float4*>(dxb + 4 * h);
                    const float dxr[4] = {dx4.x, dx4.y, dx4.z, dx4.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        acc[4 * h + r] = fmaf(f * dxr[r], float(C[r]), acc[4 * h + r]);
                        if constexpr (DUMP) {
                            const int m = 4 * h + r;
                            if (m < M && row < N) dots[(int64_t(m) * N + row) * (K >> 4) + 16 * sc + 4 * t + q] = C[r];
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const float r = sum_lane_groups(acc[m]);
            if (q == 0) pt[(m * kTileRows + n) * kWaves + wave] = r;
        }
    };
    // Outputs of a tile (wave kWaves - 1): output o = (m, row r) sums its 16 wave partials.
    // The block-dot export (DUMP) passes no Y: it writes only the dots.
    auto row_sums = [&](const float* pt, int k) __attribute__((always_inline)) {
        if constexpr (DUMP) return;
        if (wave != kWaves - 1) return;
#pragma unroll
        for (int o = lane; o < MR * kTileRows; o += 64) {
            const int m = o / kTileRows, r = o % kTileRows;
            const float4* p = reinterpret_cast<const float4*>(pt + o * kWaves);
            float s4[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 v = p[j];
                s4[j] = ((4 * j < SB ? v.x : 0.f) + (4 * j + 1 < SB ? v.y : 0.f)) +
                        ((4 * j + 2 < SB ? v.z : 0.f) + (4 * j + 3 < SB ? v.w : 0.f));
            }
            const int row = (w0 + k * G) * kTileRows + r;
            if (m < M && row < N) Y[int64_t(m) * N + row] = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        }
    };

    if (tiles > 0) {
        store(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
        issue(std::integral_constant<int, 0>{}, QD);
    }
    __syncthreads();   // tile 0 stored
    auto body = [&](auto i_c, int k) __attribute__((always_inline)) {
        constexpr int I = decltype(i_c)::value;   // k % 2
        if (active) {
            if (dword_blocks) compute(std::true_type{}, slot(std::integral_constant<int, I>{}), part[I], k);
            else compute(std::false_type{}, slot(std::integral_constant<int, I>{}), part[I], k);
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the phases apart: registers are short
        if (k > 0) row_sums(part[I ^ 1], k - 1);
        __builtin_amdgcn_sched_barrier(0);
        if (k + 1 < tiles) {
            store(std::integral_constant<int, (I + 1) % QD>{}, std::integral_constant<int, I ^ 1>{});
            issue(std::integral_constant<int, (I + 1) % QD>{}, k + 1 + QD);
        }
        __syncthreads();
    };
    int k0 = 0;
    for (; k0 + 2 <= tiles; k0 += 2) static_for<2>([&](auto i) { body(i, k0 + decltype(i)::value); });
    if (k0 < tiles) body(std::integral_constant<int, 0>{}, k0);
    if (tiles > 0) row_sums(part[(tiles - 1) & 1], tiles - 1);
}


// ------------------------------------------------------------------ wide, per-wave items, Q8_0, Q4_0, Q5_0
// The scheme of the Q4_K kernel above for Q8_0, Q4_0 and Q5_0, whose 256-value super-chunks
// are 272, 144 and 176 bytes, whole numbers of 16-byte chunks: wave w streams super-chunk w of every
// tile's 16 rows into its own LDS ring with buffer_load ... lds and computes it with the
// TiledItem of its type (four v_mfma_i32_16x16x64_i8, one per quarter of the
// super-chunk's 16-value runs).  An item's chunk c is row c / (bytes / 16), bytes
// 16 (c % (bytes / 16)) of the row's super-chunk, to slot bytes 16 c: 16-byte lanes for
// whole groups of 64 chunks, then 4-byte lanes (16 chunks per load) for the rest.
// Q8_0, Q4_0 and Q5_0 run here (on the 7B ffn_up shape Q5_0 takes 14.1 us against 16.4 us
// on the vector kernel).  The same kernel with items for Q4_1, Q5_1 and Q5_K passed the
// parity tests and ran no faster than the vector kernel (their 160- and 192-byte rows put
// several of an MFMA's 16 rows on one LDS bank, and Q5_K's unpacking is heavier), so they
// stay there.
template <int QT>
struct WideItem {
    static constexpr int kSCB = TiledItem<QT>::kSBBytes;   // bytes of one row's super-chunk
    static constexpr int kCR = kSCB / 16;                   // its 16-byte chunks
    static constexpr int kChunks = kTileRows * kCR;         // chunks of an item
    static constexpr int kFull = kChunks / 64;              // 16-byte-lane loads
    static constexpr int kTail = (kChunks % 64) / 16;       // 4-byte-lane loads
    static constexpr int kLoads = kFull + kTail;
    static constexpr int kBytes = kTileRows * kSCB;
    static_assert(kSCB % 16 == 0 && kChunks % 16 == 0, "whole chunks");
};

template <int QT, int NB>
__global__ __launch_bounds__(kThreads) void gemv_wide_kernel(const uint8_t* __restrict__ W,
                                                             const float* __restrict__ x,
                                                             float* __restrict__ y, int N, int K,
                                                             int row_bytes) {
    using WI = WideItem<QT>;
    constexpr int kIB = WI::kBytes;
    // (16 bytes past each ring: a field read as the aligned dwords around it may reach 4
    // bytes past the last wave's item)
    __shared__ __attribute__((aligned(16))) uint8_t ring0[kWaves * kIB + 16];
    __shared__ __attribute__((aligned(16))) uint8_t ring1[kWaves * kIB + 16];
    __shared__ __attribute__((aligned(16))) uint8_t ring2[NB > 2 ? kWaves * kIB + 16 : 16];
    __shared__ __attribute__((aligned(16))) uint8_t ring3[NB > 3 ? kWaves * kIB + 16 : 16];
    // x staging (digit planes [3][K], exponents per 32-block, sums per 16-run), then row
    // partials [tile][row][wave]
    __shared__ __attribute__((aligned(16))) uint8_t stage_lds[kStageBytes];
    auto slot = [&](auto b) -> uint8_t* {
        constexpr int B = decltype(b)::value;
        if constexpr (B == 0) return ring0;
        else if constexpr (B == 1) return ring1;
        else if constexpr (B == 2) return ring2;
        else return ring3;
    };
    int8_t* xp = reinterpret_cast<int8_t*>(stage_lds);
    int* ex = reinterpret_cast<int*>(stage_lds + 3 * 256 * kMaxSB);
    float* sums = reinterpret_cast<float*>(ex + 8 * kMaxSB);
    float* part = reinterpret_cast<float*>(stage_lds);
    static_assert(3 * 256 * kMaxSB + 8 * kMaxSB * 4 + 16 * kMaxSB * 4 <= kStageBytes, "x staging");

    const int SB = K >> 8;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int G = gridDim.x, w0 = blockIdx.x;
    const int TB = kTileRows * row_bytes;
    const int T = (N + kTileRows - 1) / kTileRows;
    const int tiles = (T - w0 + G - 1) / G;
    const bool active = wave < SB;

    const int nquads = K >> 2;
    float4 xe = {};
    if (tid < nquads) xe = reinterpret_cast<const float4*>(x)[tid];

    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(W), 0, N * row_bytes, kBufferWord3);
    // Idle waves issue the same loads, all past the end of the buffer (no data moves).
    auto chunk_offset = [&](int c) {
        return active ? uint32_t((c / WI::kCR) * row_bytes + wave * WI::kSCB + 16 * (c % WI::kCR)) : 0x80000000u;
    };
    // Load j of an item (at most five): 16-byte lanes for j < kFull (chunks 64 j + lane), then
    // 4-byte lanes (chunks 64 kFull + 16 (j - kFull) + lane / 4).  Written out with
    // compile-time guards: loads in a loop here make this compiler drop the kernel's
    // host-side launch stub.
    static_assert(WI::kLoads <= 5, "loads per item");
    auto load_offset = [&](int j) {
        return j < WI::kFull ? chunk_offset(64 * j + lane)
                             : chunk_offset(64 * WI::kFull + 16 * (j - WI::kFull) + (lane >> 2)) + 4 * (lane & 3);
    };
    const uint32_t vo0 = load_offset(0), vo1 = load_offset(1), vo2 = load_offset(2), vo3 = load_offset(3),
                   vo4 = load_offset(4);
    auto load = [&](uint8_t* dst, uint32_t off, auto j_c) {
        constexpr int j = decltype(j_c)::value, F = WI::kFull;
        if constexpr (j < F)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(dst + 1024 * j), 16, off, 0, 0, 0);
        else if constexpr (j < WI::kLoads)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (lds_void*)(dst + 1024 * F + 256 * (j - F)), 4, off, 0, 0, 0);
    };
    auto issue = [&](auto b, int k) {
        uint8_t* dst = slot(b) + wave * kIB;
        const uint32_t base = uint32_t((w0 + k * G) * TB);
        load(dst, base + vo0, std::integral_constant<int, 0>{});
        load(dst, base + vo1, std::integral_constant<int, 1>{});
        load(dst, base + vo2, std::integral_constant<int, 2>{});
        load(dst, base + vo3, std::integral_constant<int, 3>{});
        load(dst, base + vo4, std::integral_constant<int, 4>{});
    };
    asm volatile("s_barrier" ::: "memory");   // every wave's x requested before any weights
    static_for<NB - 1>([&](auto b) { issue(b, decltype(b)::value); });

    // Stage x: digit planes, an exponent per 32-block and the f32 sum of every 16-run.
    if (tid < nquads) {   // uniform per wave: K is a multiple of 256
        const float4 v = xe;
        float am = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
        am = lanes8_max(am);
        const int k = kFracBits - __builtin_amdgcn_frexp_expf(am);
        uint32_t d0, d1, d2;
        transpose3(digits3(v.x, k), digits3(v.y, k), digits3(v.z, k), digits3(v.w, k), d0, d1, d2);
        *reinterpret_cast<uint32_t*>(xp + 4 * tid) = d0;
        *reinterpret_cast<uint32_t*>(xp + K + 4 * tid) = d1;
        *reinterpret_cast<uint32_t*>(xp + 2 * K + 4 * tid) = d2;
        float sm = (v.x + v.y) + (v.z + v.w);
        sm = lanes8_sum<2>(sm);
        if ((tid & 3) == 0) sums[tid >> 2] = sm;
        if ((tid & 7) == 0) ex[tid >> 3] = -k;
    }
    wait_barrier<(NB - 1) * WI::kLoads>();   // x staged; the weight loads stay in flight

    const int sc = active ? wave : 0;
    const int n = lane & 15, q = lane >> 4;
    v4i a[4];
    int e[4];
    float sx[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        a[t] = v4i{0, 0, 0, 0};
        if ((n >> 2) == q && (n & 3) < 3)
            a[t] = *reinterpret_cast<const v4i*>(xp + (n & 3) * K + 256 * sc + 64 * t + 16 * q);
        e[t] = ex[8 * sc + 2 * t + (q >> 1)];
        sx[t] = sums[16 * sc + 4 * t + q];
    }
    wait_barrier<(NB - 1) * WI::kLoads>();   // x no longer read: its LDS now takes the partials

    auto compute = [&](const uint8_t* it, int k) {
        const float r = sum_lane_groups(TiledItem<QT>::run(it + n * WI::kSCB, 0, q, a, e, sx));
        if (q == 0) part[(k * kTileRows + n) * kWaves + wave] = r;
    };
    constexpr int kInFlight = (NB - 1) * WI::kLoads;
    static_assert(kInFlight < 16, "vmcnt immediate");
    auto step = [&](auto b, int k) {
        constexpr int B = decltype(b)::value;
        issue(std::integral_constant<int, (B + NB - 1) % NB>{}, k + NB - 1);
        __builtin_amdgcn_s_waitcnt(kInFlight | 0x0F70);
        compute(slot(b) + wave * kIB, k);
    };
    if (active) {
        int k0 = 0;
        for (; k0 + NB <= tiles; k0 += NB) static_for<NB>([&](auto b) { step(b, k0 + decltype(b)::value); });
        static_for<NB>([&](auto b) {
            if (k0 + decltype(b)::value < tiles) step(b, k0 + decltype(b)::value);
        });
    }
    wait_barrier<0>();

    const int wl = SB < kWaves ? SB : kWaves;
    const int r = tid >> 2, j = tid & 3;
    float s = 0.f;
    if (r < tiles * kTileRows) {
        const float4 v = *reinterpret_cast<const float4*>(part + r * kWaves + 4 * j);
        s = ((4 * j < wl ? v.x : 0.f) + (4 * j + 1 < wl ? v.y : 0.f)) +
            ((4 * j + 2 < wl ? v.z : 0.f) + (4 * j + 3 < wl ? v.w : 0.f));
    }
    s = lanes8_sum<2>(s);
    if (j == 0 && r < tiles * kTileRows) {
        const int row = (w0 + (r / kTileRows) * G) * kTileRows + r % kTileRows;
        if (row < N) y[row] = s;
    }
}

// Ring slots per type: two (one item in flight while the other is computed) where the 160 KB
// of LDS hold them next to the x staging.  As for Q4_K, a third slot was measured slower
// (Q4_0 on the 7B ffn_up shape: 10.9 us with two slots, 12.0 with three).
template <int QT>
constexpr int wide_ring() {
    constexpr int fit = (163840 - kStageBytes - 4 * 16) / (kWaves * WideItem<QT>::kBytes);
    return fit >= 2 ? 2 : fit;
}

template <int QT>
const void* wide_instance() {
    constexpr int nb = wide_ring<QT>();
    return reinterpret_cast<const void*>(gemv_wide_kernel<QT, nb>);
}

const void* wide_kernel(int type) {
    switch (type) {
        case kQ8_0: return wide_instance<kQ8_0>();
        case kQ4_0: return wide_instance<kQ4_0>();
        case kQ5_0: return wide_instance<kQ5_0>();
        default: return nullptr;
    }
}

// Ring slots per wave: three (two items in flight while the wave computes a third) once a
// workgroup has at least four tiles, else two.  Only the first item is requested before the
// x staging, the others right after it; issued all before it, deeper rings lost what they
// gained (7B ffn_up 18944 x 3584: 9.7 us with two slots, 9.8 with three, 10.9 with four),
// as every wave's items had to be accepted by the memory pipeline before the staging
// barrier.  With the later issue three slots take ffn_up from 9.41 to 9.19 us and 37888 x
// 3584 from 16.24 to 15.71 us; at two tiles per workgroup (8192 x 3584) they cost 0.3 us.
constexpr int kRing = 2;
constexpr int kRingDeep = 3;
constexpr int kRingDeepTiles = 4;   // tiles per workgroup from which the deeper ring is taken

struct Plan {
    int grid = 0;
};

Plan plan(int64_t N, int64_t K, int cu_count) {
    Plan p;
    if (N <= 0 || K % 256 || K / 256 < kMinSB || K / 256 > kMaxSB || cu_count <= 0) return p;
    const int64_t T = (N + kTileRows - 1) / kTileRows;
    const int64_t grid = T < cu_count ? T : cu_count;
    const int64_t row_bytes = (K / 256) * 144;
    // 32-bit buffer offsets: the last prefetch reaches kRingDeep rounds of tiles past the end
    if ((T + grid - 1) / grid > kMaxTilesPerGroup ||
        (T + (kRingDeep + 1) * grid) * kTileRows * row_bytes >= (int64_t(1) << 31))
        return p;
    p.grid = int(grid);
    return p;
}

// Long rows: more than 16 super-blocks and between 8 and 16 rows per CU (one tile of TR rows
// per workgroup).
int long_tile_rows(int64_t N, int64_t K, int cu_count) {
    if (N <= 0 || K % 256 || K / 256 <= kMaxSB || cu_count <= 0) return 0;
    const int64_t tr = (N + cu_count - 1) / cu_count;
    if (tr < 8 || tr > kTileRows) return 0;
    if (N * ((K / 256) * 144) > int64_t(kPastEnd)) return 0;
    return int(tr);
}

// One tile ahead in registers: two were measured slower (the Q6_K vocab head 152064 x 3584:
// 76.3 against 81.8 us; 8192 x 3584: 8.6 against 9.8 us), as with the per-wave rings above.
constexpr int kTiledDepth = 1;

int tiled_sb_bytes(int type) { return type == kQ6_K ? TiledItem<kQ6_K>::kSBBytes : 0; }

// Instances for the chunks per lane that rows of kMinSB .. kMaxSB super-chunks need.
template <int QT, int CPL>
const void* tiled_instance() {
    constexpr int lo = (kMinSB * TiledItem<QT>::kSBBytes + kThreads - 1) / kThreads;
    constexpr int hi = (kMaxSB * TiledItem<QT>::kSBBytes + kThreads - 1) / kThreads;
    if constexpr (CPL >= lo && CPL <= hi) return reinterpret_cast<const void*>(gemv_tiled_kernel<QT, kTiledDepth, CPL>);
    return nullptr;
}

template <int QT>
const void* tiled_kernel(int cpl) {
    switch (cpl) {
        case 2: return tiled_instance<QT, 2>();
        case 3: return tiled_instance<QT, 3>();
        case 4: return tiled_instance<QT, 4>();
        case 5: return tiled_instance<QT, 5>();
        default: return nullptr;
    }
}

const void* tiled_kernel_for(int type, int cpl) { return type == kQ6_K ? tiled_kernel<kQ6_K>(cpl) : nullptr; }

template <int MR, bool DUMP>
const void* q8_q6k_kernel(int cpl) {
    switch (cpl) {
        case 3: return reinterpret_cast<const void*>(gemv_q8_q6k_kernel<MR, DUMP, 3>);
        case 4: return reinterpret_cast<const void*>(gemv_q8_q6k_kernel<MR, DUMP, 4>);
        default: return nullptr;
    }
}

}  // namespace

bool gemv_tiled_applies(int type, BlockLayout layout, const uint8_t* W, int64_t N, int64_t K, int cu_count) {
    // GGUF layout, 16-byte aligned matrix, at least two 16-row tiles per CU, 12 to 16
    // super-chunks per row, the matrix ending on a 16-byte boundary (the last chunk is
    // read whole), and 32-bit buffer offsets.
    const int sbb = tiled_sb_bytes(type);
    if (sbb == 0 || layout.stride != sbb * block_values_of(type) / 256 || layout.off != 0) return false;
    if (reinterpret_cast<uintptr_t>(W) & 15) return false;
    if (N <= 0 || K % 256 || K / 256 < kMinSB || K / 256 > kMaxSB || cu_count <= 0) return false;
    if (N < 2 * kTileRows * int64_t(cu_count)) return false;
    const int64_t bytes = N * (K / 256) * sbb;
    return bytes % 16 == 0 && bytes < int64_t(kTiledPastEnd) - int64_t(kTileRows) * kMaxSB * sbb;
}

hipError_t launch_gemv_tiled(int type, const uint8_t* W, const float* x, float* y, int64_t N, int64_t K,
                             int cu_count, hipStream_t s, const char** name) {
    const int64_t T = (N + kTileRows - 1) / kTileRows;
    const int grid = int(T < cu_count ? T : cu_count);
    int n = int(N), k = int(K), row_bytes = int((K / 256) * tiled_sb_bytes(type));
    const void* f = tiled_kernel_for(type, (row_bytes + kThreads - 1) / kThreads);   // chunks per lane
    if (!f) return hipErrorInvalidValue;
    *name = "gemv_mfma<q6_K>";
    void* args[] = {&W, &x, &y, &n, &k, &row_bytes};
    return hipLaunchKernel(f, dim3(grid), dim3(kThreads), args, 0, s);
}

bool gemv_q8_tiled_applies(int type, BlockLayout layout, const uint8_t* W, const int8_t* codes, int64_t M,
                           int64_t N, int64_t K, int cu_count) {
    return type == kQ6_K && M >= 1 && M <= 8 && !(reinterpret_cast<uintptr_t>(codes) & 15) &&
           gemv_tiled_applies(type, layout, W, N, K, cu_count);
}

hipError_t launch_gemv_q8_tiled(int type, const uint8_t* W, const int8_t* codes, const float* xs, float* Y,
                                int32_t* dots, int64_t M, int64_t N, int64_t K, int cu_count, hipStream_t s,
                                const char** name) {
    if (type != kQ6_K) return hipErrorInvalidValue;
    const int64_t T = (N + kTileRows - 1) / kTileRows;
    const int grid = int(T < cu_count ? T : cu_count);
    int m = int(M), n = int(N), k = int(K), row_bytes = int((K / 256) * TiledItem<kQ6_K>::kSBBytes);
    const int cpl = (row_bytes + kThreads - 1) / kThreads;
    const bool dump = dots != nullptr;
    const void* f = M <= 4 ? (dump ? q8_q6k_kernel<4, true>(cpl) : q8_q6k_kernel<4, false>(cpl))
                           : (dump ? q8_q6k_kernel<8, true>(cpl) : q8_q6k_kernel<8, false>(cpl));
    if (!f) return hipErrorInvalidValue;
    *name = "gemv_q8_mfma<q6_K>";
    void* args[] = {&W, &codes, &xs, &Y, &dots, &m, &n, &k, &row_bytes};
    return hipLaunchKernel(f, dim3(grid), dim3(kThreads), args, 0, s);
}


namespace {


int wide_scb(int type) {
    switch (type) {
        case kQ8_0: return WideItem<kQ8_0>::kSCB;
        case kQ4_0: return WideItem<kQ4_0>::kSCB;
        case kQ5_0: return WideItem<kQ5_0>::kSCB;
        default: return 0;
    }
}

}  // namespace

bool gemv_wide_applies(int type, BlockLayout layout, const uint8_t* W, int64_t N, int64_t K, int cu_count) {
    // GGUF layout, 16-byte aligned matrix, 12 to 16 super-chunks per row, at least two and
    // at most kMaxTilesPerGroup 16-row tiles per CU, and 32-bit buffer offsets (the last
    // prefetch reaches up to five rounds of tiles past the end).
    const int scb = wide_scb(type);
    if (scb == 0 || layout.stride != scb * block_values_of(type) / 256 || layout.off != 0) return false;
    if (reinterpret_cast<uintptr_t>(W) & 15) return false;
    if (N <= 0 || K % 256 || K / 256 < kMinSB || K / 256 > kMaxSB || cu_count <= 0) return false;
    if (N < 2 * kTileRows * int64_t(cu_count)) return false;
    const int64_t T = (N + kTileRows - 1) / kTileRows;
    const int64_t grid = T < cu_count ? T : cu_count;
    const int64_t row_bytes = (K / 256) * scb;
    return (T + grid - 1) / grid <= kMaxTilesPerGroup && (T + 5 * grid) * kTileRows * row_bytes < (int64_t(1) << 31);
}

hipError_t launch_gemv_wide(int type, const uint8_t* W, const float* x, float* y, int64_t N, int64_t K,
                            int cu_count, hipStream_t s, const char** name) {
    const int64_t T = (N + kTileRows - 1) / kTileRows;
    const int grid = int(T < cu_count ? T : cu_count);
    int n = int(N), k = int(K), row_bytes = int((K / 256) * wide_scb(type));
    const void* f = wide_kernel(type);
    switch (type) {
        case kQ8_0: *name = "gemv_mfma<q8_0>"; break;
        case kQ4_0: *name = "gemv_mfma<q4_0>"; break;
        case kQ5_0: *name = "gemv_mfma<q5_0>"; break;
        default: return hipErrorInvalidValue;
    }
    void* args[] = {&W, &x, &y, &n, &k, &row_bytes};
    return hipLaunchKernel(f, dim3(grid), dim3(kThreads), args, 0, s);
}

hipError_t launch_gemv_row_tiled(const uint8_t* W, const float* x, float* y, int64_t N, int64_t K, hipStream_t s,
                                 const char** name) {
    // (the callers check row_tiled_k(K) and K <= MQ_MAX_K: a row-tiled matrix of N <= 2^24
    // rows then ends below kPastEnd only while N * row bytes does, which is checked here)
    const size_t nbytes = row_tiled_bytes(N, K);
    if (!row_tiled_k(K) || nbytes > size_t(kPastEnd)) return hipErrorInvalidValue;
    *name = "gemv_mfma_long<q4_K row-tiled>";
    const int tr = row_tile_rows(N);
    int n = int(N), k = int(K), row_bytes = int((K / 256) * 144), t = tr, nb = int(nbytes);
    void* args[] = {&W, &x, &y, &n, &k, &row_bytes, &t, &nb};
    return hipLaunchKernel(reinterpret_cast<const void*>(gemv_mfma_q4k_long_kernel<kLongRing, true>),
                           dim3(unsigned((N + tr - 1) / tr)), dim3(kThreads), args, 0, s);
}

bool gemv_mfma_applies(int type, int64_t N, int64_t K, int cu_count) {
    // Wide matrices: at least two 16-row tiles per CU; or long rows at 8..16 rows per CU.
    if (type != kQ4_K) return false;
    if (long_tile_rows(N, K, cu_count) > 0) return true;
    return N >= 2 * kTileRows * int64_t(cu_count) && plan(N, K, cu_count).grid > 0;
}

hipError_t launch_gemv_mfma(const uint8_t* W, const float* x, float* y, int64_t N, int64_t K, int cu_count,
                            hipStream_t s, const char** name) {
    if (const int tr = long_tile_rows(N, K, cu_count)) {
        *name = "gemv_mfma_long<q4_K>";
        int n = int(N), k = int(K), row_bytes = int((K / 256) * 144), t = tr, nbytes = int(N * row_bytes);
        void* args[] = {&W, &x, &y, &n, &k, &row_bytes, &t, &nbytes};
        return hipLaunchKernel(reinterpret_cast<const void*>(gemv_mfma_q4k_long_kernel<kLongRing, false>),
                               dim3(unsigned((N + tr - 1) / tr)), dim3(kThreads), args, 0, s);
    }
    const Plan p = plan(N, K, cu_count);
    if (p.grid <= 0) return hipErrorInvalidValue;
    *name = "gemv_mfma<q4_K>";
    int n = int(N), k = int(K), row_bytes = int((K / 256) * 144);
    void* args[] = {&W, &x, &y, &n, &k, &row_bytes};
    const int64_t tiles = (N + kTileRows - 1) / kTileRows;
    const void* kern = tiles >= int64_t(kRingDeepTiles) * p.grid
                           ? reinterpret_cast<const void*>(gemv_mfma_q4k_kernel<kRingDeep>)
                           : reinterpret_cast<const void*>(gemv_mfma_q4k_kernel<kRing>);
    return hipLaunchKernel(kern, dim3(p.grid),
                           dim3(kThreads), args, 0, s);
}

}  // namespace mq
