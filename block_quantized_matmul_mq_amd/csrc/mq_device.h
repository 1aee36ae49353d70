// Device-side helpers shared by the libmq kernels (gfx950, wave64).
//
// Block layouts read here ("minfer CUDA Backend Design", 2.3 fixes some sizes and
// 4.3 lists the types; the field layouts are the public GGUF ones):
//   Q8_0  34 B / 32 values : f16 d | int8 q[32]
//   Q4_0  18 B / 32 values : f16 d | 16 B nibbles (value i low, value 16 + i high nibble of byte i)
//   Q4_1  20 B / 32 values : f16 d | f16 m | 16 B nibbles
//   Q5_0  22 B / 32 values : f16 d | 4 B high bits (bit i = bit 4 of value i) | 16 B nibbles
//   Q5_1  24 B / 32 values : f16 d | f16 m | 4 B high bits | 16 B nibbles
//   Q4_K 144 B / 256 values: f16 d | f16 dmin | 12 B packed 6-bit (scale,min) x 8 | 128 B 4-bit codes
//   Q5_K 176 B / 256 values: Q4_K's 16-byte header | 32 B high bits (bit j of byte l = bit 4 of
//                            value 32 j + l) | Q4_K's 128 B of 4-bit codes
//   Q6_K 210 B / 256 values: 128 B low nibbles | 64 B high 2-bit pairs | int8 scales[16] | f16 d
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mq {

constexpr int kQ4_0 = 2;
constexpr int kQ4_1 = 3;
constexpr int kQ5_0 = 6;
constexpr int kQ5_1 = 7;
constexpr int kQ8_0 = 8;
constexpr int kQ4_K = 12;
constexpr int kQ5_K = 13;
constexpr int kQ6_K = 14;

// The 32-value types Q4_0 / Q4_1 / Q5_0 / Q5_1: block bytes, code offset (value =
// d * (code - offset) for Q4_0 / Q5_0), whether a f16 min m follows d (value =
// d * code + m) and whether 4 bytes of high bits (5-bit codes) precede the nibbles.
template <int QT> struct Legacy { static constexpr bool kIs = false; };
template <> struct Legacy<kQ4_0> { static constexpr bool kIs = true, kMin = false, kHigh = false; static constexpr int kBytes = 18, kOffset = 8; };
template <> struct Legacy<kQ4_1> { static constexpr bool kIs = true, kMin = true, kHigh = false; static constexpr int kBytes = 20, kOffset = 0; };
template <> struct Legacy<kQ5_0> { static constexpr bool kIs = true, kMin = false, kHigh = true; static constexpr int kBytes = 22, kOffset = 16; };
template <> struct Legacy<kQ5_1> { static constexpr bool kIs = true, kMin = true, kHigh = true; static constexpr int kBytes = 24, kOffset = 0; };

// Types whose value has a subtracted or added per-block minimum, carried through the
// activation block's code sum: Q4_K, Q5_K (- dmin * min_j), Q4_1, Q5_1 (+ m).
template <int QT>
constexpr bool has_min_term() {
    return QT == kQ4_K || QT == kQ5_K || QT == kQ4_1 || QT == kQ5_1;
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    // v_cvt_f32_f16: exact, subnormal halves included (f16 denormals are not flushed).
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// Byte k (0..3) of a dword as float; lowers to v_cvt_f32_ubyte{k}.
template <int k>
__device__ __forceinline__ float ubyte_f(uint32_t v) {
    return static_cast<float>((v >> (8 * k)) & 0xFFu);
}

// {hi:lo} >> (8 * sel), low 32 bits (v_alignbyte_b32).
__device__ __forceinline__ uint32_t align_byte(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_alignbyte(hi, lo, sel);
}

// A dword at an address that is only 2-byte aligned, built from the one or two
// naturally aligned dwords that contain it.  Never touches a dword that holds
// none of the requested bytes, so it cannot read past the end of a buffer.
__device__ __forceinline__ uint32_t load_u32_a2(const uint8_t* p) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uint32_t* q = reinterpret_cast<const uint32_t*>(a & ~uintptr_t(3));
    const uint32_t lo = q[0];
    if (a & 2) return align_byte(q[1], lo, 2);
    return lo;
}

__device__ __forceinline__ uint32_t load_u16(const uint8_t* p) {
    return *reinterpret_cast<const uint16_t*>(p);
}

// OCP FP6 E2M3 (1 sign, 2 exponent and 3 mantissa bits, exponent bias 1, no Inf/NaN):
// the 6-bit code of k / 2 for an integer k with |k| <= 15.  Every multiple of 1/2 up to
// 7.5 is exact in this format: 0.5 is the subnormal 4/8, 1..1.5, 2..3.5 and 4..7.5 are the
// three binades.
__device__ __forceinline__ uint32_t e2m3_half_code(int k) {
    constexpr uint64_t kLow = 0x161412100C080400ull;    // |k| = 0..7
    constexpr uint64_t kHigh = 0x1F1E1D1C1B1A1918ull;   // |k| = 8..15
    const uint32_t a = uint32_t(k < 0 ? -k : k);
    const uint64_t tbl = a < 8 ? kLow : kHigh;
    return (uint32_t(k < 0) << 5) | uint32_t((tbl >> (8 * (a & 7))) & 0x3Fu);
}

// e2m3_half_code of four 4-bit fields at once (byte i of `nib` holds field i).  SIGNED: each
// field is a two's-complement k in -8..7 (the high nibble of a signed byte), else k = 0..15.
// Two eight-entry byte lookups (v_perm_b32: selectors 0..3 pick bytes of the second
// operand, 4..7 of the first) and a third that takes, per byte, the half named by bit 3.
template <bool SIGNED>
__device__ __forceinline__ uint32_t e2m3_half_codes4(uint32_t nib) {
    constexpr uint32_t t0 = 0x0C080400u, t1 = 0x16141210u;         // k = 0..3, 4..7
    constexpr uint32_t t2 = SIGNED ? 0x32343638u : 0x1B1A1918u;    // k = -8..-5, or 8..11
    constexpr uint32_t t3 = SIGNED ? 0x24282C30u : 0x1F1E1D1Cu;    // k = -4..-1, or 12..15
    const uint32_t sel = nib & 0x07070707u;
    const uint32_t lo = __builtin_amdgcn_perm(t1, t0, sel);
    const uint32_t hi = __builtin_amdgcn_perm(t3, t2, sel);
    return __builtin_amdgcn_perm(hi, lo, ((nib >> 1) & 0x04040404u) | 0x03020100u);
}

// Reductions over aligned groups of eight lanes (every lane of the wave active): lane i
// with lanes i ^ 1 and i ^ 2 (DPP quad permutations), then with lane 7 - i of its eight
// (DPP half-row mirror), which after the first two steps holds the other quad's value.
// The result equals the xor-butterfly's over lanes i ^ 1, i ^ 2, i ^ 4 bit for bit, also
// for f32 sums: after each step the lanes of a pair or quad hold the same value, and
// each addition takes the same two operands (in either order).
template <int STEP>
__device__ __forceinline__ int dpp8_partner(int v) {
    if constexpr (STEP == 0) return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    else if constexpr (STEP == 1) return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    else return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);   // row_half_mirror
}

template <int STEP>
__device__ __forceinline__ float dpp8_partner(float v) {
    return __builtin_bit_cast(float, dpp8_partner<STEP>(__builtin_bit_cast(int, v)));
}

// over groups of four lanes (the first two steps) or eight (all three)
template <int STEPS = 3>
__device__ __forceinline__ float lanes8_max(float a) {
    a = fmaxf(a, dpp8_partner<0>(a));
    a = fmaxf(a, dpp8_partner<1>(a));
    if constexpr (STEPS == 3) a = fmaxf(a, dpp8_partner<2>(a));
    return a;
}

template <int STEPS = 3, typename T>
__device__ __forceinline__ T lanes8_sum(T s) {
    s += dpp8_partner<0>(s);
    s += dpp8_partner<1>(s);
    if constexpr (STEPS == 3) s += dpp8_partner<2>(s);
    return s;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Q4_K: 6-bit scale and min of sub-block j from the packed bytes
// s0 = bytes 0..3, s1 = bytes 4..7, s2 = bytes 8..11 of the 12-byte field.
//   j < 4 : scale = b[j] & 63,                         min = b[j+4] & 63
//   j >= 4: scale = (b[j+4] & 15) | (b[j-4] >> 6) << 4, min = (b[j+4] >> 4) | (b[j] >> 6) << 4
__device__ __forceinline__ void q4k_scale_min(uint32_t s0, uint32_t s1, uint32_t s2, int j,
                                              uint32_t& sc, uint32_t& mn) {
    if (j < 4) {
        sc = (s0 >> (8 * j)) & 63u;
        mn = (s1 >> (8 * j)) & 63u;
    } else {
        const int k = j - 4;
        const uint32_t b_hi = (s2 >> (8 * k)) & 0xFFu;
        sc = (b_hi & 15u) | (((s0 >> (8 * k + 6)) & 3u) << 4);
        mn = (b_hi >> 4) | (((s1 >> (8 * k + 6)) & 3u) << 4);
    }
}

}  // namespace mq
