// One "unit" of a weight row as the vector-ALU GEMV kernels read it: the raw bytes of
// 64 values (Q4_K, Q5_K, Q6_K) or of one 32-value block (Q8_0, Q4_0, Q4_1, Q5_0, Q5_1),
// loaded with naturally aligned 16-byte or 4-byte loads, and the code bytes unpacked from
// them.  Shared by the f32-x
// GEMV (gemv.hip) and the multi-row GEMV over quantized activations (gemv_q8.hip).
//
// A weight row is K / 64 units (Q4_K, Q5_K, Q6_K) or K / 32 units (the 32-value types).  `stride` and `off`
// place a block in memory: the GGUF payload (stride = block bytes, off = 0) or the
// repacked layout (Q6_K 224-byte slots, Q8_0 36-byte slots at offset 2).
#pragma once

#include "mq_device.h"

namespace mq {

// ---------------------------------------------------------------- Q4_K
// Unit u: super-block u/4, 64-value group c = u%4 (sub-blocks 2c and 2c+1).  Bytes: the
// 16-byte header (d, dmin, packed scales) and the 32 code bytes at 16 + 32c; byte i holds
// the code of value 64c+i (low nibble) and of value 64c+32+i (high nibble).
struct RawQ4K {
    static constexpr int kValues = 64;
    uint4 hd, q0, q1;

    __device__ void load(const uint8_t* __restrict__ row, int u, int, int) {
        const uint8_t* blk = row + 144 * (u >> 2);
        hd = *reinterpret_cast<const uint4*>(blk);
        const uint4* qs = reinterpret_cast<const uint4*>(blk + 16 + 32 * (u & 3));
        q0 = qs[0];
        q1 = qs[1];
    }
    // codes of values 0..31 (lo) and 32..63 (hi) of the unit, one per byte
    __device__ void codes(uint32_t (&lo)[8], uint32_t (&hi)[8]) const {
        const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            lo[k] = w[k] & 0x0F0F0F0Fu;
            hi[k] = (w[k] >> 4) & 0x0F0F0F0Fu;
        }
    }
    // 6-bit (scale, min) of sub-blocks 2c, 2c+1: bytes 0, 1 of scp (scales) and mnp (mins).
    // No branches: c < 2 reads bytes 2c, 2c+1 of the first two dwords; c >= 2 assembles the
    // fields from all three.
    __device__ void scale_min(int c, uint32_t& scp, uint32_t& mnp) const {
        const uint32_t sh = 16u * uint32_t(c & 1);
        const uint32_t t0 = hd.y >> sh, t1 = hd.z >> sh, t2 = hd.w >> sh;
        const uint32_t sc_hi = (t2 & 0x0F0Fu) | ((t0 >> 2) & 0x3030u);
        const uint32_t mn_hi = ((t2 >> 4) & 0x0F0Fu) | ((t1 >> 2) & 0x3030u);
        scp = c >= 2 ? sc_hi : (t0 & 0x3F3Fu);
        mnp = c >= 2 ? mn_hi : (t1 & 0x3F3Fu);
    }
    __device__ float d() const { return half_bits_to_float(hd.x & 0xFFFFu); }
    __device__ float dmin() const { return half_bits_to_float(hd.x >> 16); }
};

// ---------------------------------------------------------------- Q6_K
// Unit u: super-block u/4, half h = (u/2)%2, lane run l in [l0, l0+16) with l0 = 16*(u%2):
// values 128h + 32t + l for t < 4 (16 each, one sub-scale each).  Low 4 bits: ql[64h + l]
// (t = 0 low nibble, t = 2 high nibble) and ql[64h + 32 + l] (t = 1, 3); high 2 bits: bits
// 2t..2t+1 of qh[32h + l].  GGUF blocks are 210 bytes, so a block starts on a 2-byte
// boundary: every segment is read as naturally aligned dwords and realigned with
// v_alignbyte (a no-op in the 16-byte-aligned 224-byte slots of the repacked layout).
struct RawQ6K {
    static constexpr int kValues = 64;
    uint32_t a[5], b[5], hq[5], s[3];
    uint32_t dbits;
    uint32_t shift;

    __device__ void load(const uint8_t* __restrict__ row, int u, int stride, int off) {
        const uint8_t* blk = row + stride * (u >> 2) + off;
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
    // realigned segments: A, B (the two ql runs), H (qh run), s0/s1 (the half's 8 sub-scales)
    __device__ void realign(uint32_t (&A)[4], uint32_t (&B)[4], uint32_t (&H)[4], uint32_t& s0,
                            uint32_t& s1) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            A[i] = align_byte(a[i + 1], a[i], shift);
            B[i] = align_byte(b[i + 1], b[i], shift);
            H[i] = align_byte(hq[i + 1], hq[i], shift);
        }
        s0 = align_byte(s[1], s[0], shift);
        s1 = align_byte(s[2], s[1], shift);
    }
    // the 16 codes (0..63, one per byte) of run t
    __device__ static void run_codes(int t, const uint32_t (&A)[4], const uint32_t (&B)[4], const uint32_t (&H)[4],
                                     uint32_t (&code)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t ql = (t & 1) ? B[i] : A[i];
            const uint32_t lo = (t < 2) ? ql : (ql >> 4);
            const uint32_t hb = (H[i] >> (2 * t)) & 0x03030303u;
            code[i] = (lo & 0x0F0F0F0Fu) | (hb << 4);
        }
    }
    // signed sub-scale of run t of unit u (byte 2t + u%2 of the half's eight)
    __device__ static float subscale(int t, int u, uint32_t s0, uint32_t s1) {
        const int g = 2 * t + (u & 1);
        const uint32_t word = g < 4 ? s0 : s1;
        return float(int32_t(word << (24 - 8 * (g & 3))) >> 24);
    }
    __device__ float d() const { return half_bits_to_float(dbits); }
};

// ---------------------------------------------------------------- Q8_0
// Unit u = block u (34 bytes: f16 d, 32 int8 codes), 2-byte aligned in the GGUF payload
// (at offset 2 of a 36-byte slot in the repacked layout, so that its codes are 4-byte
// aligned).
struct RawQ80 {
    static constexpr int kValues = 32;
    uint32_t w[9];
    uint32_t odd;

    __device__ void load(const uint8_t* __restrict__ row, int u, int stride, int off) {
        const uintptr_t base = reinterpret_cast<uintptr_t>(row + stride * u + off);
        odd = uint32_t(base & 2);
        const uint32_t* p = reinterpret_cast<const uint32_t*>(base & ~uintptr_t(3));
        // 9 naturally aligned dwords cover the block; each holds a byte of it
#pragma unroll
        for (int i = 0; i < 9; ++i) w[i] = p[i];
    }
    __device__ void codes(uint32_t (&c)[8]) const {
#pragma unroll
        for (int i = 0; i < 8; ++i) c[i] = odd ? w[i + 1] : align_byte(w[i + 1], w[i], 2);
    }
    __device__ float d() const { return half_bits_to_float(odd ? (w[0] >> 16) : (w[0] & 0xFFFFu)); }
};

// ---------------------------------------------------------------- Q5_K
// Unit u: super-block u/4, 64-value group c = u%4 (sub-blocks 2c and 2c+1), as Q4_K, plus
// the 32 bytes of high bits: bit 2c (2c+1) of byte l is bit 4 of the code of value 64c + l
// (64c + 32 + l).  176-byte blocks are 16-byte aligned.
struct RawQ5K {
    static constexpr int kValues = 64;
    uint4 hd, q0, q1, h0, h1;

    __device__ void load(const uint8_t* __restrict__ row, int u, int, int) {
        const uint8_t* blk = row + 176 * (u >> 2);
        hd = *reinterpret_cast<const uint4*>(blk);
        h0 = *reinterpret_cast<const uint4*>(blk + 16);
        h1 = *reinterpret_cast<const uint4*>(blk + 32);
        const uint4* qs = reinterpret_cast<const uint4*>(blk + 48 + 32 * (u & 3));
        q0 = qs[0];
        q1 = qs[1];
    }
    // 5-bit codes of values 0..31 (lo) and 32..63 (hi) of unit u, one per byte
    __device__ void codes(int u, uint32_t (&lo)[8], uint32_t (&hi)[8]) const {
        const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
        const uint32_t h[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
        const uint32_t s = 2u * uint32_t(u & 3);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            lo[k] = (w[k] & 0x0F0F0F0Fu) | (((h[k] >> s) & 0x01010101u) << 4);
            hi[k] = ((w[k] >> 4) & 0x0F0F0F0Fu) | (((h[k] >> (s + 1)) & 0x01010101u) << 4);
        }
    }
    // 6-bit (scale, min) of sub-blocks 2c, 2c+1 (the Q4_K header packing)
    __device__ void scale_min(int c, uint32_t& scp, uint32_t& mnp) const {
        const uint32_t sh = 16u * uint32_t(c & 1);
        const uint32_t t0 = hd.y >> sh, t1 = hd.z >> sh, t2 = hd.w >> sh;
        const uint32_t sc_hi = (t2 & 0x0F0Fu) | ((t0 >> 2) & 0x3030u);
        const uint32_t mn_hi = ((t2 >> 4) & 0x0F0Fu) | ((t1 >> 2) & 0x3030u);
        scp = c >= 2 ? sc_hi : (t0 & 0x3F3Fu);
        mnp = c >= 2 ? mn_hi : (t1 & 0x3F3Fu);
    }
    __device__ float d() const { return half_bits_to_float(hd.x & 0xFFFFu); }
    __device__ float dmin() const { return half_bits_to_float(hd.x >> 16); }
};

// ---------------------------------------------------------------- Q4_0 / Q4_1 / Q5_0 / Q5_1
// Unit u = block u (32 values).  Q4_0 and Q5_0 blocks (18 and 22 bytes) start on a 2-byte
// boundary, Q4_1 and Q5_1 blocks (20 and 24 bytes) on a 4-byte one: the block is read as the
// naturally aligned dwords that cover it (each holds at least one of its bytes) and every
// field is realigned from them with v_alignbyte.
// Bit i of four bits -> bit 0 of byte i (no carries: the shifted copies do not overlap).
__device__ __forceinline__ uint32_t spread4(uint32_t v) { return (v * 0x00204081u) & 0x01010101u; }

template <int QT>
struct RawLegacy {
    using L = Legacy<QT>;
    static constexpr int kValues = 32;
    static constexpr bool kAligned4 = L::kBytes % 4 == 0;                // block starts 4-byte aligned
    static constexpr int kWords = (L::kBytes + (kAligned4 ? 0 : 2) + 3) / 4;
    static constexpr int kQh = L::kMin ? 4 : 2;                           // byte offset of qh
    static constexpr int kQs = kQh + (L::kHigh ? 4 : 0);                  // byte offset of the nibbles
    uint32_t w[kWords];
    uint32_t odd;   // 2 when the block starts 2 bytes into a dword

    __device__ void load(const uint8_t* __restrict__ row, int u, int, int) {
        const uintptr_t base = reinterpret_cast<uintptr_t>(row + L::kBytes * u);
        odd = kAligned4 ? 0u : uint32_t(base & 2);
        const uint32_t* p = reinterpret_cast<const uint32_t*>(base & ~uintptr_t(3));
#pragma unroll
        for (int i = 0; i < kWords; ++i) w[i] = p[i];
    }
    // the 4 block bytes from byte `pos` (even) of the block
    template <int pos>
    __device__ uint32_t at() const {
        const uint32_t even = (pos % 4 == 0) ? w[pos / 4] : align_byte(w[pos / 4 + 1], w[pos / 4], 2);
        if constexpr (kAligned4) return even;
        constexpr int q = pos + 2;   // the same bytes when the block starts 2 bytes in
        const uint32_t shifted = (q % 4 == 0) ? w[q / 4] : align_byte(w[q / 4 + 1], w[q / 4], 2);
        return odd ? shifted : even;
    }
    // codes of values 0..15 (c[0..3]) and 16..31 (c[4..7]), one per byte (0..15, or 0..31 with qh)
    __device__ void codes(uint32_t (&c)[8]) const {
        const uint32_t q[4] = {at<kQs>(), at<kQs + 4>(), at<kQs + 8>(), at<kQs + 12>()};
        uint32_t qh = 0;
        if constexpr (L::kHigh) qh = at<kQh>();
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            c[k] = q[k] & 0x0F0F0F0Fu;
            c[k + 4] = (q[k] >> 4) & 0x0F0F0F0Fu;
            if constexpr (L::kHigh) {
                c[k] |= spread4((qh >> (4 * k)) & 15u) << 4;
                c[k + 4] |= spread4((qh >> (16 + 4 * k)) & 15u) << 4;
            }
        }
    }
    __device__ float d() const {
        const uint32_t h = kAligned4 ? w[0] : (odd ? (w[0] >> 16) : w[0]);
        return half_bits_to_float(h & 0xFFFFu);
    }
    __device__ float m() const {
        if constexpr (L::kMin) return half_bits_to_float(w[0] >> 16);   // 4-byte aligned types only
        return 0.f;
    }
};

}  // namespace mq
