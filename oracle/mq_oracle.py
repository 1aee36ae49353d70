"""Plain numpy oracle for GGUF block-quantized matmul (TEST INFRASTRUCTURE).

Only the tests, the smoke check and bench.py's CPU-baseline leg use this
module.  It shares nothing with the HIP library.

Everything here is a direct definition: decode each block to f64 values, then
take ordinary products and sums.  Floating point is f64 except where the
method itself fixes f32 (the activation quantizer, whose integer codes must be
reproduced bit for bit).

Sources (page title, section):

* "minfer CUDA Backend Design", 2.3 Weight residency and registry -- a Q4_K
  payload is exactly od*(id/256)*144 bytes (row-major: output rows, then
  256-value super-blocks along the input dimension); q8_0 is 34 bytes per 32
  values; the Q6_K block is repacked into 224-byte slots, so its raw block is
  smaller than 224 bytes.
* "minfer CUDA Backend Design", 4.3 Eligibility -- a quantized matmul needs
  the input dimension to be a multiple of 32.
* "minfer CUDA Backend Design", 4.4 Execution dispatch -- decode uses int dot
  products over q8_0-quantized activations; prefill uses the int8 MMQ GEMM
  over a pre-quantized activation plane.
* "minfer Architecture Execution Plan", C4 S2b design decision 4 (and
  "minfer CUDA Backend Design", 4.7) -- the Q8_0 quantizer: amax over the
  32-block, scale = amax/127, codes rounded half to even.

Readings where the pages are silent:

* R1  Block bit layouts (d/dmin/scales/qs for Q4_K; ql/qh/scales/d for Q6_K;
      d then q[32] for Q8_0) are the public GGUF layouts.  The pages give only
      sizes.  GGUF interop is parity unpinned (no GGUF file is available).
* R2  Q6_K is 128 (ql) + 64 (qh) + 16 (int8 scales) + 2 (f16 d) = 210 bytes.
* R3  Q6_K sub-scales are signed int8.
* R4  The activation scale is f32: d = f32(amax) / f32(127), IEEE division.
* R5  Codes are round-half-to-even of the IEEE f32 quotient x / d (a true
      division, not a multiply by 1/d), clamped to [-127, 127]; a block with
      amax == 0 has d == 0 and all codes 0.
* R6  The per-block code sum S = sum(q) is part of the quantized activation
      (it carries the Q4_K min term through the int path).
* R7  Block dots are exact integers: per 32-value block for Q8_0 and Q4_K
      (Q4_K codes in [0, 15], unsigned), per 16-value group for Q6_K with the
      signed code (c - 32).
* R14 The 32-value types Q4_0 / Q4_1 / Q5_0 / Q5_1 (named by the matmul type
      whitelist, "minfer CUDA Backend Design", 4.3 Eligibility; Q4_0's 18 bytes
      per 32 values by the bytes-per-element ratio it shares with Q4_K, same
      page, 2.3) use the public GGUF layouts: f16 d, then (Q4_1, Q5_1) f16 m,
      then (Q5_0, Q5_1) 4 bytes of high bits qh, then 16 bytes of nibbles.
      Value i < 16 is the low nibble of byte i, value 16 + i its high nibble;
      bit i of the little-endian 32-bit qh is bit 4 of value i's code.
      Q4_0: d * (code - 8); Q5_0: d * (code - 16); Q4_1, Q5_1: d * code + m.
      Sizes 18, 20, 22, 24 bytes.
* R15 Q5_K (176 bytes per 256 values, the block size "GPU Safety (Metal + CUDA
      Backends)", 3. Audit findings, names as the bound of the kernel's qh/qs
      reads): Q4_K's
      header (f16 d, f16 dmin, the same 12 packed bytes of 6-bit scales and
      mins), then 32 bytes qh, then Q4_K's 128 bytes of nibbles; bit j of
      qh[e % 32] is bit 4 of the code of value e, j = e // 32 its sub-block.
      value_e = d * scale_j * code_e - dmin * min_j, codes in [0, 31].
* R16 Block dots of the new types are per 32-value block: the signed code
      (code - 8 or code - 16) for Q4_0 / Q5_0, the unsigned code for Q4_1,
      Q5_1 and Q5_K (whose min term rides on the activation block's code sum).
* R17 Q4_K's repacked layout is a pre-decoded plane for the prefill product (the
      pages' reference pre-decodes weight planes at load time for a faster
      prefill, "minfer CUDA Backend Design", 2.3): per 64-value step t and weight
      row n (rows padded with zeros to a multiple of 256), each of the step's two
      32-value sub-blocks as a 24-byte record of its codes c, each the 6-bit OCP
      FP6 E2M3 code of c / 2 (exact), value i at bits 6i..6i+5, plus the bf16
      hi/lo split of its scale d*sc and of its min -dmin*m.  The quantized
      activation plane carries the matching section: each code q as the E2M3
      codes of h / 2 and l / 2 with q = 16 h + l, h = q >> 4, l = q & 15, and the
      bf16 hi/lo splits of dx and of dx * S (f32 product).  The byte layouts are
      ``repack`` (Q4_K) and ``act_f6_section`` below; the products on the plane
      are checked against ``mmq`` (the plane holds the scales to 16 bits, well
      inside the 2e-4 tolerance).
* R18 Q4_K's row-tiled layout (a second derived layout, for the decode GEMV of
      long rows; the pages admit derived layouts behind an exact-length gate,
      "minfer CUDA Backend Design", 2.3): rows are taken in groups of
      R = min(16, ceil(N / 256)) consecutive rows, the last group filled with
      zero rows; a group stores its rows' super-block 0 blocks one after
      another (row order), then their super-block 1 blocks, and so on; groups
      follow in order.  Whole 144-byte blocks move, unchanged.  Only for rows
      of more than 16 super-blocks.
* R12 The repacked layout (the one-time device-layout transform): the pages
      repack a Q6_K block into a 16-byte-aligned 224-byte slot ("minfer CUDA
      Backend Design", 2.3); the block sits at the start of its slot and the
      14 trailing bytes are zero.  A Q8_0 block goes to a 36-byte slot at
      offset 2, the first 2 bytes zero, so that its 32 codes start 4-byte
      aligned (the pages name no Q8_0 repack: this layout is a reading).
      Rows and blocks keep their order.
"""

import numpy as np

# GGUF tensor-type ids.
Q4_0 = 2
Q4_1 = 3
Q5_0 = 6
Q5_1 = 7
Q8_0 = 8
Q4_K = 12
Q5_K = 13
Q6_K = 14

BLOCK_VALUES = {Q4_0: 32, Q4_1: 32, Q5_0: 32, Q5_1: 32, Q8_0: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256}
BLOCK_BYTES = {Q4_0: 18, Q4_1: 20, Q5_0: 22, Q5_1: 24, Q8_0: 34, Q4_K: 144, Q5_K: 176, Q6_K: 210}

# R14: the 32-value types -- (has a min m, has high bits qh, code offset of the _0 types)
LEGACY = {Q4_0: (False, False, 8), Q4_1: (True, False, 0), Q5_0: (False, True, 16), Q5_1: (True, True, 0)}

ACT_BLOCK = 32


def row_bytes(qtype, K):
    """Bytes of one weight row of K values (K a multiple of the block size)."""
    bv = BLOCK_VALUES[qtype]
    if K % bv:
        raise ValueError(f"K={K} is not a multiple of {bv}")
    return (K // bv) * BLOCK_BYTES[qtype]


def f16_bits_to_f64(lo_byte, hi_byte):
    """IEEE binary16 (little-endian byte pair) -> f64, exactly.

    Written from the binary16 definition (1 sign, 5 exponent, 10 fraction
    bits; exponent 0 is subnormal), not via numpy's float16, so that it is a
    second implementation next to the library conversion used by the tests.
    Inf/NaN encodings are outside the contract and raise.
    """
    bits = lo_byte.astype(np.int64) | (hi_byte.astype(np.int64) << 8)
    sign = np.where(bits >> 15, -1.0, 1.0)
    exp = (bits >> 10) & 0x1F
    frac = (bits & 0x3FF).astype(np.float64)
    if np.any(exp == 0x1F):
        raise ValueError("f16 Inf/NaN scale in a weight block")
    normal = sign * (1.0 + frac / 1024.0) * np.exp2(exp.astype(np.float64) - 15.0)
    subnormal = sign * frac * 2.0 ** -24
    return np.where(exp == 0, subnormal, normal)


# R12: slot bytes and the block's offset inside its slot, per repackable type.
REPACK_SLOT = {Q8_0: (36, 2), Q6_K: (224, 0)}


def repack(raw, qtype, N, K):
    """R12: the repacked bytes (uint8, N * K/bv slots) of a GGUF payload.

    Block b of row n goes to slot b of row n at the slot's offset; every other
    byte of the slot is zero.  Pinned by the page's 224-byte Q6_K slot
    (tests/golden/block_sizes.txt), the alignment each slot is for, and a
    per-block brute force.  Q4_K goes to its MMQ plane instead (R17,
    ``q4_k_plane``).
    """
    if qtype == Q4_K:
        return q4_k_plane(raw, N, K)
    slot, off = REPACK_SLOT[qtype]
    b = _blocks(raw, qtype, N, K)
    out = np.zeros((N, b.shape[1], slot), dtype=np.uint8)
    out[:, :, off:off + BLOCK_BYTES[qtype]] = b
    return out.reshape(-1)


def unpack_repacked(rep, qtype, N, K):
    """Inverse of repack: the GGUF payload back from the repacked bytes.

    Raises ValueError when the size is not exact or a padding byte is nonzero.
    """
    slot, off = REPACK_SLOT[qtype]
    nb = K // BLOCK_VALUES[qtype]
    rep = np.ascontiguousarray(rep, dtype=np.uint8).reshape(-1)
    if rep.size != N * nb * slot:
        raise ValueError(f"repacked payload is {rep.size} bytes, expected exactly {N * nb * slot}")
    r = rep.reshape(N, nb, slot)
    pad = np.concatenate([r[:, :, :off], r[:, :, off + BLOCK_BYTES[qtype]:]], axis=-1)
    if np.any(pad):
        raise ValueError("nonzero padding byte in a repacked slot")
    return np.ascontiguousarray(r[:, :, off:off + BLOCK_BYTES[qtype]]).reshape(-1)


# ---------------------------------------------------------------- R18: row tiles

def row_tile_rows(N):
    """R18: rows per group of Q4_K's row-tiled layout."""
    return min(16, -(-N // 256))


def q4_k_row_tiled(raw, N, K):
    """R18: Q4_K's row-tiled layout (uint8) of a GGUF payload.

    Pinned by a block-by-block construction on small matrices, by the inverse
    ``unpack_q4_k_row_tiled`` (a loop over the groups) and by the group sizes
    the layout states (tests/test_oracle_row_tiled.py).
    """
    SB = K // 256
    if K % 256 or SB <= 16:
        raise ValueError(f"the row-tiled layout is for rows of more than 16 super-blocks (K={K})")
    R = row_tile_rows(N)
    G = -(-N // R)
    b = np.zeros((G * R, SB, 144), dtype=np.uint8)
    b[:N] = _blocks(raw, Q4_K, N, K)
    # [group, row in group, super-block, byte] -> [group, super-block, row in group, byte]
    return np.ascontiguousarray(b.reshape(G, R, SB, 144).transpose(0, 2, 1, 3)).reshape(-1)


def unpack_q4_k_row_tiled(rep, N, K):
    """Inverse of q4_k_row_tiled: the GGUF payload back (raises on a wrong size or a
    nonzero byte in the filler rows)."""
    SB = K // 256
    R = row_tile_rows(N)
    G = -(-N // R)
    rep = np.ascontiguousarray(rep, dtype=np.uint8).reshape(-1)
    if rep.size != G * R * SB * 144:
        raise ValueError(f"row-tiled payload is {rep.size} bytes, expected exactly {G * R * SB * 144}")
    out = np.zeros((N, SB, 144), dtype=np.uint8)
    for g in range(G):
        grp = rep[g * R * SB * 144:(g + 1) * R * SB * 144].reshape(SB, R, 144)
        for r in range(R):
            n = g * R + r
            if n < N:
                out[n] = grp[:, r, :]
            elif np.any(grp[:, r, :]):
                raise ValueError("nonzero byte in a filler row of the row-tiled layout")
    return out.reshape(-1)


# ---------------------------------------------------------------- R17: the fp6 planes

PLANE_ROWS = 256       # weight rows of the Q4_K plane are padded to a multiple of this
ACT_PLANE_ROWS = 128   # activation rows of the fp6 section are padded to a multiple of this


def e2m3_value(code):
    """Value of a 6-bit OCP FP6 E2M3 code: sign bit 5, exponent bits 4..3 (bias 1),
    mantissa bits 2..0; exponent 0 is subnormal (m / 8), else 2^(e-1) * (1 + m/8)."""
    code = int(code)
    sign = -1.0 if code & 32 else 1.0
    e, m = (code >> 3) & 3, code & 7
    return sign * (m / 8.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 8.0))


def e2m3_code_of_half(k):
    """The E2M3 code whose value is k / 2 (integer k, |k| <= 15; +0 for k = 0): the
    unique code with that value, found by search over the format's codes."""
    k = int(k)
    if k == 0:
        return 0
    for code in range(64):
        if e2m3_value(code) == k / 2.0:
            return code
    raise ValueError(f"{k}/2 is not an E2M3 value")


def fp6_records(codes6):
    """Pack 6-bit codes [..., 32] into 24-byte records [..., 24]: value i at bits 6i..6i+5
    of the little-endian 192-bit record."""
    codes6 = np.asarray(codes6, dtype=np.uint8)
    bits = ((codes6[..., :, None] >> np.arange(6, dtype=np.uint8)) & 1).reshape(codes6.shape[:-1] + (192,))
    return np.packbits(bits, axis=-1, bitorder="little")


def bf16_hilo(x):
    """bf16 hi/lo split of f32 values: hi = bf16(x), lo = bf16(x - hi), each rounded to
    nearest with ties to even; returned as uint16 bit patterns (hi, lo)."""
    def rne(v):
        b = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
        return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)
    x = np.asarray(x, dtype=np.float32)
    hi = rne(x)
    hi_f = (hi.astype(np.uint32) << 16).view(np.float32)
    lo = rne((x - hi_f).astype(np.float32))
    return hi, lo


def _dwords(lo16, hi16):
    """uint32 words lo16 | hi16 << 16."""
    return np.asarray(lo16, dtype=np.uint32) | (np.asarray(hi16, dtype=np.uint32) << 16)


def _le_bytes(words):
    """uint32 words [..., w] -> their little-endian bytes [..., 4 w]."""
    w = np.ascontiguousarray(words, dtype="<u4")
    return w.view(np.uint8).reshape(w.shape[:-1] + (4 * w.shape[-1],))


def q4_k_plane(raw, N, K):
    """R17: Q4_K's repacked layout (uint8), the plane of the fp6 prefill product.

    Np = N rounded up to PLANE_ROWS; T = K / 64 steps of 80 * Np bytes.  In step t,
    for the two sub-blocks b = 2t + u (u = 0, 1) of each row n < N (rows n >= N are zero):
      bytes 16 (u Np + n) ..          bytes 0..15 of the 24-byte E2M3 record of c / 2
      bytes 32 Np + 8 (u Np + n) ..   bytes 16..23 of that record
      bytes 48 Np + 8 (u Np + n) ..   words (dw_hi | dw_hi << 16, dw_lo | dw_lo << 16)
      bytes 64 Np + 8 (u Np + n) ..   words (mw_hi | mw_lo << 16) twice
    with dw = d * sc_b and mw = -dmin * m_b (both exact in f32) split by bf16_hilo.
    """
    if K % 256:
        raise ValueError(f"K={K} is not a multiple of 256")
    d, dmin, sc, mn, codes = q4_k_fields(raw, N, K)
    KB, T = K // 32, K // 64
    Np = -(-N // PLANE_ROWS) * PLANE_ROWS
    table = np.array([e2m3_code_of_half(c) for c in range(16)], dtype=np.uint8)
    rec = np.zeros((Np, KB, 24), dtype=np.uint8)
    rec[:N] = fp6_records(table[codes.reshape(N, KB, 32)])
    dw = np.zeros((Np, KB), dtype=np.float32)
    mw = np.zeros((Np, KB), dtype=np.float32)
    dw[:N] = (d[..., None] * sc).reshape(N, KB).astype(np.float32)
    mw[:N] = (-(dmin[..., None] * mn)).reshape(N, KB).astype(np.float32)
    dh, dl = bf16_hilo(dw)
    mh, ml = bf16_hilo(mw)
    outer = _le_bytes(np.stack([_dwords(dh, dh), _dwords(dl, dl)], axis=-1))   # [Np, KB, 8]
    mwin = _le_bytes(np.stack([_dwords(mh, ml), _dwords(mh, ml)], axis=-1))
    out = np.zeros((T, 80 * Np), dtype=np.uint8)
    for t in range(T):
        slab = out[t]
        for u in range(2):
            b = 2 * t + u
            slab[16 * u * Np:16 * (u + 1) * Np] = rec[:, b, :16].reshape(-1)
            slab[32 * Np + 8 * u * Np:32 * Np + 8 * (u + 1) * Np] = rec[:, b, 16:].reshape(-1)
            slab[48 * Np + 8 * u * Np:48 * Np + 8 * (u + 1) * Np] = outer[:, b].reshape(-1)
            slab[64 * Np + 8 * u * Np:64 * Np + 8 * (u + 1) * Np] = mwin[:, b].reshape(-1)
    return out.reshape(-1)


def act_f6_section(q, d, S):
    """R17: the fp6 section of the quantized activation plane (uint8) for the codes q
    [M, K], scales d [M, K/32] and code sums S [M, K/32] of ``quantize_act``.

    Mp = M rounded up to ACT_PLANE_ROWS; T = ceil(K / 64) steps of 128 * Mp bytes.  In
    step t, for blocks b = 2t + u of each row m < M (rows m >= M, and a block past the
    row's end when K % 64 == 32, are zero), with q = 16 h + l, h = q >> 4, l = q & 15:
      bytes 16 ((2u + g) Mp + m) ..          bytes 0..15 of the E2M3 record of h / 2 (g = 0)
                                             or l / 2 (g = 1)
      bytes 64 Mp + 8 ((2u + g) Mp + m) ..   bytes 16..23 of it
      bytes 96 Mp + 8 (u Mp + m) ..          words (dx_hi | dx_lo << 16) twice
      bytes 112 Mp + 8 (u Mp + m) ..         words (tx_hi | tx_hi << 16, tx_lo | tx_lo << 16)
    with tx = dx * S the f32 product, both split by bf16_hilo.
    """
    q = np.asarray(q, dtype=np.int8).astype(np.int64)
    M, K = q.shape
    KB = K // 32
    T = -(-K // 64)
    Mp = -(-M // ACT_PLANE_ROWS) * ACT_PLANE_ROWS
    table = {k: e2m3_code_of_half(k) for k in range(-15, 16)}
    enc = np.vectorize(lambda k: table[int(k)], otypes=[np.uint8])
    qb = q.reshape(M, KB, 32)
    recs = np.zeros((2, Mp, 2 * T, 24), dtype=np.uint8)
    recs[0, :M, :KB] = fp6_records(enc(qb >> 4))
    recs[1, :M, :KB] = fp6_records(enc(qb & 15))
    dx = np.zeros((Mp, 2 * T), dtype=np.float32)
    tx = np.zeros((Mp, 2 * T), dtype=np.float32)
    dx[:M, :KB] = np.asarray(d, dtype=np.float32)
    tx[:M, :KB] = (np.asarray(d, dtype=np.float32) * np.asarray(S, dtype=np.int32).astype(np.float32)).astype(np.float32)
    xh, xl = bf16_hilo(dx)
    th, tl = bf16_hilo(tx)
    outer = _le_bytes(np.stack([_dwords(xh, xl), _dwords(xh, xl)], axis=-1))
    mins = _le_bytes(np.stack([_dwords(th, th), _dwords(tl, tl)], axis=-1))
    out = np.zeros((T, 128 * Mp), dtype=np.uint8)
    for t in range(T):
        slab = out[t]
        for u in range(2):
            b = 2 * t + u
            for g in range(2):
                sp = 2 * u + g
                slab[16 * sp * Mp:16 * (sp + 1) * Mp] = recs[g, :, b, :16].reshape(-1)
                slab[64 * Mp + 8 * sp * Mp:64 * Mp + 8 * (sp + 1) * Mp] = recs[g, :, b, 16:].reshape(-1)
            slab[96 * Mp + 8 * u * Mp:96 * Mp + 8 * (u + 1) * Mp] = outer[:, b].reshape(-1)
            slab[112 * Mp + 8 * u * Mp:112 * Mp + 8 * (u + 1) * Mp] = mins[:, b].reshape(-1)
    return out.reshape(-1)


def _blocks(raw, qtype, N, K):
    raw = np.ascontiguousarray(raw, dtype=np.uint8).reshape(-1)
    nbytes = N * row_bytes(qtype, K)
    if raw.size != nbytes:
        raise ValueError(f"payload is {raw.size} bytes, expected exactly {nbytes}")
    nb = K // BLOCK_VALUES[qtype]
    return raw.reshape(N, nb, BLOCK_BYTES[qtype])


def q8_0_fields(raw, N, K):
    """Q8_0 fields: d f64 [N, nb] and signed codes int64 [N, nb, 32].

    Block (34 bytes): f16 d at bytes 0..1, then 32 int8 codes (R1).
    value_i = d * q_i.
    """
    b = _blocks(raw, Q8_0, N, K)
    d = f16_bits_to_f64(b[..., 0], b[..., 1])
    q = b[..., 2:34].astype(np.int8).astype(np.int64)
    return d, q


def q4_k_fields(raw, N, K):
    """Q4_K fields: d, dmin f64 [N, nb]; sc, m int64 [N, nb, 8]; codes int64 [N, nb, 256].

    Block (144 bytes, R1): f16 d (bytes 0-1), f16 dmin (2-3), 12 bytes of
    packed 6-bit (scale, min) pairs for the eight 32-value sub-blocks (4-15),
    then 128 bytes of 4-bit codes (16-143).

    Sub-block j's 6-bit scale and min, with b = the 12 packed bytes:
      j < 4 : scale = low 6 bits of b[j],   min = low 6 bits of b[j+4]
      j >= 4: scale = low nibble of b[j+4]  plus the top 2 bits of b[j-4] as bits 4-5
              min   = high nibble of b[j+4] plus the top 2 bits of b[j]   as bits 4-5
    Codes: value e lies in 64-value chunk c = e // 64 at offset r = e % 64;
    its code is the low nibble of qs[32c + r] when r < 32, else the high
    nibble of qs[32c + r - 32].
    value_e = d * scale_j * code_e - dmin * min_j, with j = e // 32.
    """
    b = _blocks(raw, Q4_K, N, K)
    d, dmin, sc, mn = _k_header(b)
    codes = _k_nibbles(b[..., 16:144].astype(np.int64))
    return d, dmin, sc, mn, codes


def _k_header(b):
    """d, dmin and the eight 6-bit (scale, min) pairs of a Q4_K / Q5_K block header."""
    d = f16_bits_to_f64(b[..., 0], b[..., 1])
    dmin = f16_bits_to_f64(b[..., 2], b[..., 3])
    s = b[..., 4:16].astype(np.int64)
    sc = np.empty(s.shape[:-1] + (8,), dtype=np.int64)
    mn = np.empty_like(sc)
    for j in range(4):
        sc[..., j] = s[..., j] & 63
        mn[..., j] = s[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (s[..., j + 4] & 15) | ((s[..., j - 4] >> 6) << 4)
        mn[..., j] = (s[..., j + 4] >> 4) | ((s[..., j] >> 6) << 4)
    return d, dmin, sc, mn


def _k_nibbles(qs):
    """The 256 4-bit codes of 128 K-quant code bytes (chunk c: low nibbles, then high)."""
    codes = np.empty(qs.shape[:-1] + (256,), dtype=np.int64)
    for c in range(4):
        chunk = qs[..., 32 * c:32 * c + 32]
        codes[..., 64 * c:64 * c + 32] = chunk & 15
        codes[..., 64 * c + 32:64 * c + 64] = chunk >> 4
    return codes


def q5_k_fields(raw, N, K):
    """Q5_K fields (R15): d, dmin f64 [N, nb]; sc, m int64 [N, nb, 8]; codes int64 [N, nb, 256] in [0, 31].

    Block (176 bytes): Q4_K's 16-byte header (bytes 0-15), qh (16-47), then
    the 128 nibble bytes (48-175) read as in Q4_K; bit j = e // 32 of
    qh[e % 32] is bit 4 of the code of value e.
    value_e = d * scale_j * code_e - dmin * min_j.
    """
    b = _blocks(raw, Q5_K, N, K)
    d, dmin, sc, mn = _k_header(b)
    qh = b[..., 16:48].astype(np.int64)
    low = _k_nibbles(b[..., 48:176].astype(np.int64))
    high = np.empty_like(low)
    for j in range(8):
        high[..., 32 * j:32 * j + 32] = (qh >> j) & 1
    return d, dmin, sc, mn, low | (high << 4)


def legacy_fields(raw, qtype, N, K):
    """Q4_0 / Q4_1 / Q5_0 / Q5_1 fields (R14): d, m f64 [N, nb]; codes int64 [N, nb, 32].

    m is 0 for Q4_0 / Q5_0.  Returns (d, m, codes, offset) with
    value_i = d * (code_i - offset) + m (offset 8 for Q4_0, 16 for Q5_0, else 0).
    """
    has_min, has_high, offset = LEGACY[qtype]
    b = _blocks(raw, qtype, N, K)
    d = f16_bits_to_f64(b[..., 0], b[..., 1])
    pos = 2
    m = np.zeros_like(d)
    if has_min:
        m = f16_bits_to_f64(b[..., 2], b[..., 3])
        pos = 4
    codes = np.zeros(b.shape[:-1] + (32,), dtype=np.int64)
    if has_high:
        qh = b[..., pos:pos + 4].astype(np.int64)
        bits = qh[..., 0] | (qh[..., 1] << 8) | (qh[..., 2] << 16) | (qh[..., 3] << 24)
        for i in range(32):
            codes[..., i] = ((bits >> i) & 1) << 4
        pos += 4
    qs = b[..., pos:pos + 16].astype(np.int64)
    codes[..., 0:16] |= qs & 15
    codes[..., 16:32] |= qs >> 4
    return d, m, codes, offset


def q6_k_fields(raw, N, K):
    """Q6_K fields: d f64 [N, nb]; scales int64 [N, nb, 16]; codes int64 [N, nb, 256] in [0, 63].

    Block (210 bytes, R1/R2): 128 bytes ql (low 4 bits of each code), 64 bytes
    qh (high 2 bits), 16 signed int8 sub-scales (one per 16 values, R3), f16 d.
    For value e: half h = e // 128, r = e % 128, quarter t = r // 32,
    l = r % 32.  Low 4 bits: ql[64h + l + 32*(t % 2)], low nibble for t < 2,
    high nibble for t >= 2.  High 2 bits: bits 2t..2t+1 of qh[32h + l].
    value_e = d * scales[e // 16] * (code_e - 32).
    """
    b = _blocks(raw, Q6_K, N, K)
    ql = b[..., 0:128].astype(np.int64)
    qh = b[..., 128:192].astype(np.int64)
    scales = b[..., 192:208].astype(np.int8).astype(np.int64)
    d = f16_bits_to_f64(b[..., 208], b[..., 209])
    codes = np.empty(b.shape[:-1] + (256,), dtype=np.int64)
    for h in range(2):
        for t in range(4):
            low_src = ql[..., 64 * h + 32 * (t % 2): 64 * h + 32 * (t % 2) + 32]
            low = (low_src >> (4 * (t // 2))) & 15
            high = (qh[..., 32 * h: 32 * h + 32] >> (2 * t)) & 3
            e0 = 128 * h + 32 * t
            codes[..., e0:e0 + 32] = low | (high << 4)
    return d, scales, codes


def decode(raw, qtype, N, K):
    """O1: deq(W) as f64 [N, K] (exact: every value is a short product of f16 and small ints)."""
    if qtype == Q8_0:
        d, q = q8_0_fields(raw, N, K)
        w = d[..., None] * q
    elif qtype == Q4_K:
        d, dmin, sc, mn, codes = q4_k_fields(raw, N, K)
        sub_scale = np.repeat(d[..., None] * sc, 32, axis=-1)
        sub_min = np.repeat(dmin[..., None] * mn, 32, axis=-1)
        w = sub_scale * codes - sub_min
    elif qtype == Q6_K:
        d, scales, codes = q6_k_fields(raw, N, K)
        group_scale = np.repeat(d[..., None] * scales, 16, axis=-1)
        w = group_scale * (codes - 32)
    elif qtype == Q5_K:
        d, dmin, sc, mn, codes = q5_k_fields(raw, N, K)
        sub_scale = np.repeat(d[..., None] * sc, 32, axis=-1)
        sub_min = np.repeat(dmin[..., None] * mn, 32, axis=-1)
        w = sub_scale * codes - sub_min
    elif qtype in LEGACY:
        d, m, codes, offset = legacy_fields(raw, qtype, N, K)
        w = d[..., None] * (codes - offset) + m[..., None]
    else:
        raise ValueError(f"unsupported type {qtype}")
    return w.reshape(N, K)


def gemv(raw, qtype, x, N, K, row_chunk=4096):
    """O2: y[n] = sum_k deq(W)[n, k] * x[k] in f64 (x f32 promoted exactly).

    Decodes in row chunks so a large weight (e.g. a vocab head) fits in memory.
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64).reshape(K)
    raw = np.ascontiguousarray(raw, dtype=np.uint8).reshape(N, row_bytes(qtype, K))
    y = np.empty(N, dtype=np.float64)
    for r0 in range(0, N, row_chunk):
        r1 = min(N, r0 + row_chunk)
        y[r0:r1] = decode(raw[r0:r1], qtype, r1 - r0, K) @ x64
    return y


def quantize_act(X):
    """O3: per row, per 32-value block: amax, d = amax/127 in f32, q = rne(x/d).

    Returns (q int8 [M, K], d f32 [M, K/32], S int32 [M, K/32]) with S the sum
    of the block's codes (R4-R6).  All arithmetic that decides a code is IEEE
    f32, as the method fixes it.
    """
    X = np.asarray(X, dtype=np.float32)
    M, K = X.shape
    if K % ACT_BLOCK:
        raise ValueError(f"K={K} is not a multiple of {ACT_BLOCK}")
    xb = X.reshape(M, K // ACT_BLOCK, ACT_BLOCK)
    amax = np.max(np.abs(xb), axis=-1)
    d = (amax / np.float32(127.0)).astype(np.float32)
    safe_d = np.where(d > 0, d, np.float32(1.0)).astype(np.float32)
    ratio = (xb / safe_d[..., None]).astype(np.float32)
    q = np.clip(np.rint(ratio), -127, 127)
    q = np.where(d[..., None] > 0, q, 0).astype(np.int8)
    S = q.astype(np.int32).sum(axis=-1, dtype=np.int32)
    return q.reshape(M, K), d, S


def block_dots(raw, qtype, q, N, K):
    """O4: exact int64 block dot products between weight codes and activation codes.

    * Q8_0: D[m, n, b] = sum_{i<32} qw[n, 32b+i] * qx[m, 32b+i]
    * Q4_K: D[m, n, b] = sum_{i<32} code[n, 32b+i] * qx[m, 32b+i]   (codes 0..15)
    * Q6_K: D[m, n, g] = sum_{i<16} (code[n, 16g+i] - 32) * qx[m, 16g+i]
    * Q4_0, Q5_0: per 32-block, the signed code (code - 8, code - 16)
    * Q4_1, Q5_1, Q5_K: per 32-block, the unsigned code (R16)
    """
    q = np.asarray(q, dtype=np.int8).astype(np.int64)
    M = q.shape[0]
    if qtype == Q8_0:
        _, wq = q8_0_fields(raw, N, K)
        grp = 32
    elif qtype == Q4_K:
        wq = q4_k_fields(raw, N, K)[4]
        grp = 32
    elif qtype == Q6_K:
        wq = q6_k_fields(raw, N, K)[2] - 32
        grp = 16
    elif qtype == Q5_K:
        wq = q5_k_fields(raw, N, K)[4]
        grp = 32
    elif qtype in LEGACY:
        _, _, codes, offset = legacy_fields(raw, qtype, N, K)
        wq = codes - offset
        grp = 32
    else:
        raise ValueError(f"unsupported type {qtype}")
    wq = wq.reshape(N, K // grp, grp)
    xq = q.reshape(M, K // grp, grp)
    return np.einsum("ngi,mgi->mng", wq, xq)


def mmq(raw, qtype, q, d, N, K):
    """O5: Y[m, n] = sum_k deq(W)[n, k] * dx[m, k//32] * qx[m, k] in f64.

    The activation is the dequantized q8 value x_hat = dx * qx (exact in f64).
    """
    q = np.asarray(q, dtype=np.int8).astype(np.float64)
    d = np.asarray(d, dtype=np.float32).astype(np.float64)
    M = q.shape[0]
    x_hat = (q.reshape(M, K // 32, 32) * d[..., None]).reshape(M, K)
    return x_hat @ decode(raw, qtype, N, K).T


def mmq_from_block_dots(raw, qtype, q, d, S, N, K):
    """O5 in block-dot form (what an int path accumulates), f64.

    * Q8_0: Y = sum_b dx[m,b] * d[n,b] * D[m,n,b]
    * Q4_K: Y = sum_j dx[m,j] * (d*sc_j * D[m,n,j] - dmin*m_j * S[m,j])
    * Q6_K: Y = sum_g dx[m,g//2] * d*s_g * D[m,n,g]
    * Q5_K: as Q4_K (5-bit codes)
    * Q4_0, Q5_0: Y = sum_b dx[m,b] * d[n,b] * D[m,n,b]   (signed codes)
    * Q4_1, Q5_1: Y = sum_b dx[m,b] * (d[n,b] * D[m,n,b] + m[n,b] * S[m,b])
    Tests check that this equals ``mmq`` to ~1e-15 relative.
    """
    D = block_dots(raw, qtype, q, N, K).astype(np.float64)
    dx = np.asarray(d, dtype=np.float32).astype(np.float64)
    if qtype == Q8_0:
        dw, _ = q8_0_fields(raw, N, K)
        return np.einsum("mb,nb,mnb->mn", dx, dw.reshape(N, K // 32), D)
    if qtype in (Q4_K, Q5_K):
        dd, dmin, sc, mn, _ = (q4_k_fields if qtype == Q4_K else q5_k_fields)(raw, N, K)
        wscale = (dd[..., None] * sc).reshape(N, K // 32)
        wmin = (dmin[..., None] * mn).reshape(N, K // 32)
        S = np.asarray(S, dtype=np.int64).astype(np.float64)
        main = np.einsum("mb,nb,mnb->mn", dx, wscale, D)
        minterm = np.einsum("mb,nb,mb->mn", dx, wmin, S)
        return main - minterm
    if qtype == Q6_K:
        dd, scales, _ = q6_k_fields(raw, N, K)
        gscale = (dd[..., None] * scales).reshape(N, K // 16)
        dxg = np.repeat(dx, 2, axis=-1)
        return np.einsum("mg,ng,mng->mn", dxg, gscale, D)
    if qtype in LEGACY:
        dw, mw, _, _ = legacy_fields(raw, qtype, N, K)
        S = np.asarray(S, dtype=np.int64).astype(np.float64)
        main = np.einsum("mb,nb,mnb->mn", dx, dw, D)
        return main + np.einsum("mb,nb,mb->mn", dx, mw, S)
    raise ValueError(f"unsupported type {qtype}")
