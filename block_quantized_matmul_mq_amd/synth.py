"""Seeded synthetic inputs: f32 weights/activations and their GGUF block encodings.

This module makes the inputs that both the HIP library and the CPU checks
consume.  It holds none of the matmul's arithmetic (no decode, no dot
product, no activation quantizer); it only draws seeded f32 tensors and
packs them into the GGUF block byte layouts Q8_0 (34 B / 32 values),
Q4_0 / Q4_1 / Q5_0 / Q5_1 (18 / 20 / 22 / 24 B / 32), Q4_K (144 B / 256),
Q5_K (176 B / 256) and Q6_K (210 B / 256).  Sizes follow "minfer CUDA
Backend Design", 2.3 Weight residency and registry; the field layouts are the
public GGUF ones.

Weight quantizers (the pages print none for the K-quants; these are the
readings used to make test weights, each with an exact error bound):

* Q8_0: d = f16_rne(amax / 127); q = clamp(rne(w / d), -127, 127), dividing
  by the stored f16 scale, so |w - d*q| <= d/2.
* Q4_K: min-max with covering rounding.  Per 32-value sub-block j:
  lo_j = min(0, min w), hi_j = max w; dmin = f16_up(max_j(-lo_j) / 63);
  m_j = ceil(-lo_j / dmin); d = f16_up(max_j(hi_j + dmin*m_j) / (15*63));
  sc_j = ceil((hi_j + dmin*m_j) / (15*d)); code = clamp(rne((w + dmin*m_j) /
  (d*sc_j)), 0, 15).  The code grid covers [lo_j, hi_j], so
  |w - (d*sc_j*code - dmin*m_j)| <= d*sc_j / 2.
* Q6_K: step_g = amax_g / 31 per 16-value group; d = f16_up(max_g step_g / 127);
  s_g = ceil(step_g / d) <= 127; code - 32 = rne(w / (d*s_g)) in [-31, 31];
  |w - d*s_g*(code - 32)| <= d*s_g / 2.
* Q4_0 / Q5_0 (symmetric, codes offset by 8 / 16): d = f16_up(amax / 7) or
  f16_up(amax / 15); q = rne(w / d) (|q| <= 7 or 15); |w - d*q| <= d/2.
* Q4_1 / Q5_1 (affine): m = f16_down(min w); d = f16_up((max w - m) / 15 or
  31); code = clamp(rne((w - m) / d), 0, 15 or 31); the grid covers
  [min w, max w], so |w - (d*code + m)| <= d/2 (a block of equal values has
  d = 0 and is off by at most its f16 rounding of m).
* Q5_K: the Q4_K quantizer with 31 code steps instead of 15.

Seeds: numpy ``default_rng(SeedSequence([0, config_index, tensor_index]))``.
"""

import numpy as np

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

_ROW_CHUNK = 2048


def rng_for(config_index, tensor_index, base=0):
    return np.random.default_rng(np.random.SeedSequence([base, config_index, tensor_index]))


def normal_f32(rng, shape, sigma=1.0):
    """f32 N(0, sigma^2), drawn in float32."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def activations(M, K, config_index, tensor_index=100, sigma=1.0):
    """Activation rows X f32 [M, K] ~ N(0, 1)."""
    return normal_f32(rng_for(config_index, tensor_index), (M, K), sigma)


def f16_round_up(v):
    """Smallest IEEE binary16 value >= v (v >= 0, finite), as a float16 array."""
    v = np.asarray(v, dtype=np.float64)
    h = v.astype(np.float16)
    low = h.astype(np.float64) < v
    h = np.where(low, np.nextafter(h, np.float16(np.inf)), h).astype(np.float16)
    if not np.all(np.isfinite(h)):
        raise ValueError("scale overflows binary16")
    return h


def f16_round_down(v):
    """Largest IEEE binary16 value <= v (finite), as a float16 array."""
    v = np.asarray(v, dtype=np.float64)
    h = v.astype(np.float16)
    high = h.astype(np.float64) > v
    h = np.where(high, np.nextafter(h, np.float16(-np.inf)), h).astype(np.float16)
    if not np.all(np.isfinite(h)):
        raise ValueError("value overflows binary16")
    return h


def _f16_bytes(h):
    return np.ascontiguousarray(h.astype("<f2")).view(np.uint8).reshape(h.shape + (2,))


def encode_q8_0(W):
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    nb = K // 32
    wb = W.reshape(N, nb, 32)
    amax = np.max(np.abs(wb), axis=-1)
    d16 = (amax / np.float32(127.0)).astype(np.float16)
    d32 = d16.astype(np.float32)
    safe = np.where(d32 > 0, d32, np.float32(1.0))
    q = np.clip(np.rint(wb / safe[..., None]), -127, 127)
    q = np.where(d32[..., None] > 0, q, 0).astype(np.int8)
    out = np.empty((N, nb, 34), dtype=np.uint8)
    out[..., 0:2] = _f16_bytes(d16)
    out[..., 2:34] = q.view(np.uint8)
    return out.reshape(N, nb * 34)


def _pack_q4_k(d, dmin, sc, mn, codes):
    """Pack fields into 144-byte blocks.  sc, mn: [.., 8] ints < 64; codes [.., 256] < 16."""
    shape = d.shape
    out = np.zeros(shape + (144,), dtype=np.uint8)
    out[..., 0:2] = _f16_bytes(d)
    out[..., 2:4] = _f16_bytes(dmin)
    sc = sc.astype(np.uint8)
    mn = mn.astype(np.uint8)
    for j in range(4):
        out[..., 4 + j] = (sc[..., j] & 63) | ((sc[..., j + 4] >> 4) << 6)
        out[..., 8 + j] = (mn[..., j] & 63) | ((mn[..., j + 4] >> 4) << 6)
        out[..., 12 + j] = (sc[..., j + 4] & 15) | ((mn[..., j + 4] & 15) << 4)
    codes = codes.astype(np.uint8)
    for c in range(4):
        lo = codes[..., 64 * c:64 * c + 32]
        hi = codes[..., 64 * c + 32:64 * c + 64]
        out[..., 16 + 32 * c:16 + 32 * c + 32] = lo | (hi << 4)
    return out


def encode_q4_k(W):
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    nb = K // 256
    out = np.empty((N, nb, 144), dtype=np.uint8)
    for r0 in range(0, N, _ROW_CHUNK):
        r1 = min(N, r0 + _ROW_CHUNK)
        wb = W[r0:r1].reshape(r1 - r0, nb, 8, 32).astype(np.float64)
        lo = np.minimum(0.0, wb.min(axis=-1))
        hi = wb.max(axis=-1)
        mprime = -lo + 0.0          # +0.0, never -0.0, for an all-positive sub-block
        dmin = f16_round_up(mprime.max(axis=-1) / 63.0)
        dmin64 = dmin.astype(np.float64)[..., None]
        mn = np.where(dmin64 > 0, np.minimum(63, np.ceil(mprime / np.where(dmin64 > 0, dmin64, 1.0))), 0)
        offset = dmin64 * mn
        span = hi + offset
        d = f16_round_up(span.max(axis=-1) / (15.0 * 63.0))
        d64 = d.astype(np.float64)[..., None]
        sc = np.where(d64 > 0, np.minimum(63, np.ceil(span / (15.0 * np.where(d64 > 0, d64, 1.0)))), 0)
        step = (d64 * sc)[..., None]
        codes = np.where(step > 0, np.clip(np.rint((wb + offset[..., None]) / np.where(step > 0, step, 1.0)), 0, 15), 0)
        out[r0:r1] = _pack_q4_k(d, dmin, sc.astype(np.int64), mn.astype(np.int64),
                                codes.reshape(r1 - r0, nb, 256).astype(np.int64))
    return out.reshape(N, nb * 144)


def _k_quant_header_codes(wb, steps):
    """The Q4_K covering quantizer with `steps` code steps (15 for Q4_K, 31 for Q5_K).

    wb: f64 [.., nb, 8, 32].  Returns d, dmin (f16 [.., nb]), sc, mn (int [.., nb, 8]) and
    codes (int [.., nb, 256]).
    """
    lo = np.minimum(0.0, wb.min(axis=-1))
    hi = wb.max(axis=-1)
    mprime = -lo + 0.0
    dmin = f16_round_up(mprime.max(axis=-1) / 63.0)
    dmin64 = dmin.astype(np.float64)[..., None]
    mn = np.where(dmin64 > 0, np.minimum(63, np.ceil(mprime / np.where(dmin64 > 0, dmin64, 1.0))), 0)
    offset = dmin64 * mn
    span = hi + offset
    d = f16_round_up(span.max(axis=-1) / (steps * 63.0))
    d64 = d.astype(np.float64)[..., None]
    sc = np.where(d64 > 0, np.minimum(63, np.ceil(span / (steps * np.where(d64 > 0, d64, 1.0)))), 0)
    step = (d64 * sc)[..., None]
    codes = np.where(step > 0, np.clip(np.rint((wb + offset[..., None]) / np.where(step > 0, step, 1.0)), 0, steps), 0)
    shape = wb.shape[:-2]
    return d, dmin, sc.astype(np.int64), mn.astype(np.int64), codes.reshape(shape + (256,)).astype(np.int64)


def encode_q5_k(W):
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    nb = K // 256
    out = np.empty((N, nb, 176), dtype=np.uint8)
    for r0 in range(0, N, _ROW_CHUNK):
        r1 = min(N, r0 + _ROW_CHUNK)
        wb = W[r0:r1].reshape(r1 - r0, nb, 8, 32).astype(np.float64)
        d, dmin, sc, mn, codes = _k_quant_header_codes(wb, 31)
        out[r0:r1] = _pack_q5_k(d, dmin, sc, mn, codes)
    return out.reshape(N, nb * 176)


def _pack_q5_k(d, dmin, sc, mn, codes):
    """176-byte blocks: the Q4_K header and nibbles around 32 bytes of high bits."""
    q4 = _pack_q4_k(d, dmin, sc, mn, codes & 15)
    out = np.zeros(d.shape + (176,), dtype=np.uint8)
    out[..., 0:16] = q4[..., 0:16]
    out[..., 48:176] = q4[..., 16:144]
    high = (codes >> 4).astype(np.uint8)
    for j in range(8):
        out[..., 16:48] |= high[..., 32 * j:32 * j + 32] << j
    return out


def _pack_legacy(qtype, d, m, codes):
    """Blocks of the 32-value types: f16 d, [f16 m], [qh], 16 nibble bytes; codes [.., 32]."""
    nbytes = BLOCK_BYTES[qtype]
    out = np.zeros(d.shape + (nbytes,), dtype=np.uint8)
    out[..., 0:2] = _f16_bytes(d)
    pos = 2
    if qtype in (Q4_1, Q5_1):
        out[..., 2:4] = _f16_bytes(m)
        pos = 4
    codes = codes.astype(np.int64)
    if qtype in (Q5_0, Q5_1):
        bits = np.zeros(d.shape, dtype=np.int64)
        for i in range(32):
            bits |= ((codes[..., i] >> 4) & 1) << i
        for k in range(4):
            out[..., pos + k] = (bits >> (8 * k)) & 0xFF
        pos += 4
    out[..., pos:pos + 16] = ((codes[..., 0:16] & 15) | ((codes[..., 16:32] & 15) << 4)).astype(np.uint8)
    return out


def _encode_legacy(qtype, W):
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    nb = K // 32
    wb = W.reshape(N, nb, 32).astype(np.float64)
    top = 15 if qtype in (Q4_0, Q4_1) else 31
    if qtype in (Q4_0, Q5_0):
        qmax, off = (7, 8) if qtype == Q4_0 else (15, 16)
        d = f16_round_up(np.max(np.abs(wb), axis=-1) / qmax)
        d64 = d.astype(np.float64)[..., None]
        q = np.where(d64 > 0, np.clip(np.rint(wb / np.where(d64 > 0, d64, 1.0)), -qmax, qmax), 0)
        codes = q + off
        m = np.zeros_like(d)
    else:
        m = f16_round_down(wb.min(axis=-1))
        m64 = m.astype(np.float64)[..., None]
        d = f16_round_up((wb.max(axis=-1) - m.astype(np.float64)) / top)
        d64 = d.astype(np.float64)[..., None]
        codes = np.where(d64 > 0, np.clip(np.rint((wb - m64) / np.where(d64 > 0, d64, 1.0)), 0, top), 0)
    return _pack_legacy(qtype, d, m, codes).reshape(N, nb * BLOCK_BYTES[qtype])


def _pack_q6_k(d, scales, codes):
    """Pack fields into 210-byte blocks.  scales [.., 16] int8; codes [.., 256] in [0, 63]."""
    shape = d.shape
    out = np.zeros(shape + (210,), dtype=np.uint8)
    codes = codes.astype(np.uint8)
    for h in range(2):
        for t in range(4):
            c = codes[..., 128 * h + 32 * t:128 * h + 32 * t + 32]
            ql_lo = 64 * h + 32 * (t % 2)
            out[..., ql_lo:ql_lo + 32] |= (c & 15) << (4 * (t // 2))
            out[..., 128 + 32 * h:128 + 32 * h + 32] |= ((c >> 4) & 3) << (2 * t)
    out[..., 192:208] = scales.astype(np.int8).view(np.uint8)
    out[..., 208:210] = _f16_bytes(d)
    return out


def encode_q6_k(W):
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    nb = K // 256
    out = np.empty((N, nb, 210), dtype=np.uint8)
    for r0 in range(0, N, _ROW_CHUNK):
        r1 = min(N, r0 + _ROW_CHUNK)
        wb = W[r0:r1].reshape(r1 - r0, nb, 16, 16).astype(np.float64)
        step = np.max(np.abs(wb), axis=-1) / 31.0
        d = f16_round_up(step.max(axis=-1) / 127.0)
        d64 = d.astype(np.float64)[..., None]
        s = np.where(d64 > 0, np.minimum(127, np.ceil(step / np.where(d64 > 0, d64, 1.0))), 0)
        gs = (d64 * s)[..., None]
        c = np.where(gs > 0, np.clip(np.rint(wb / np.where(gs > 0, gs, 1.0)), -31, 31), 0) + 32
        out[r0:r1] = _pack_q6_k(d, s.astype(np.int64), c.reshape(r1 - r0, nb, 256).astype(np.int64))
    return out.reshape(N, nb * 210)


ENCODERS = {Q8_0: encode_q8_0, Q4_K: encode_q4_k, Q6_K: encode_q6_k, Q5_K: encode_q5_k,
            Q4_0: lambda W: _encode_legacy(Q4_0, W), Q4_1: lambda W: _encode_legacy(Q4_1, W),
            Q5_0: lambda W: _encode_legacy(Q5_0, W), Q5_1: lambda W: _encode_legacy(Q5_1, W)}


def weights_f32(N, K, config_index, tensor_index, sigma=0.02, rows=None):
    """Seeded W f32 ~ N(0, sigma^2).  Row chunk c (of 2048 rows) draws from
    SeedSequence([0, config_index, tensor_index, c]), so any row range can be
    regenerated on its own.  ``rows`` = (r0, r1) returns just that range."""
    r0, r1 = rows if rows is not None else (0, N)
    out = np.empty((r1 - r0, K), dtype=np.float32)
    for c in range(r0 // _ROW_CHUNK, (r1 + _ROW_CHUNK - 1) // _ROW_CHUNK):
        c0, c1 = c * _ROW_CHUNK, min(N, (c + 1) * _ROW_CHUNK)
        rng = np.random.default_rng(np.random.SeedSequence([0, config_index, tensor_index, c]))
        chunk = normal_f32(rng, (c1 - c0, K), sigma)
        lo, hi = max(c0, r0), min(c1, r1)
        out[lo - r0:hi - r0] = chunk[lo - c0:hi - c0]
    return out


def quantized_weight(qtype, N, K, config_index, tensor_index, sigma=0.02, threads=8):
    """Seeded W (see weights_f32) encoded to uint8 [N, row_bytes], chunk by chunk
    on a thread pool (numpy releases the GIL); memory stays bounded for a
    vocab-sized head and the bytes do not depend on the thread count."""
    from concurrent.futures import ThreadPoolExecutor
    enc = ENCODERS[qtype]
    starts = list(range(0, N, _ROW_CHUNK))

    def one(r0):
        r1 = min(N, r0 + _ROW_CHUNK)
        return enc(weights_f32(N, K, config_index, tensor_index, sigma, rows=(r0, r1)))

    with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
        parts = list(ex.map(one, starts))
    return np.concatenate(parts, axis=0)


def _random_f16(rng, shape, exp_lo, exp_hi, allow_negative=True):
    """Finite f16 values with exponents in [exp_lo, exp_hi] (unbiased), random sign."""
    e = rng.integers(exp_lo, exp_hi + 1, size=shape)
    m = rng.integers(0, 1024, size=shape)
    v = (1.0 + m / 1024.0) * np.exp2(e.astype(np.float64))
    if allow_negative:
        v = v * np.where(rng.integers(0, 2, size=shape) == 1, -1.0, 1.0)
    return v.astype(np.float16)


def random_blocks(qtype, N, K, rng, exp_lo=-14, exp_hi=-4):
    """Arbitrary block bytes (every code/scale field uniformly random) with finite f16 scales.

    Exercises fields a quantizer never emits: Q4_K scale/min up to 63 with any
    top bits, negative Q6_K sub-scales, negative d, subnormal-free d.
    """
    nb = K // BLOCK_VALUES[qtype]
    raw = rng.integers(0, 256, size=(N, nb, BLOCK_BYTES[qtype]), dtype=np.uint8)
    if qtype == Q8_0:
        raw[..., 0:2] = _f16_bytes(_random_f16(rng, (N, nb), exp_lo, exp_hi))
        # -128 is not a code the quantizer emits but it is a valid int8: keep it.
    elif qtype in (Q4_K, Q5_K, Q4_1, Q5_1):
        raw[..., 0:2] = _f16_bytes(_random_f16(rng, (N, nb), exp_lo, exp_hi))
        raw[..., 2:4] = _f16_bytes(_random_f16(rng, (N, nb), exp_lo, exp_hi))
    elif qtype in (Q4_0, Q5_0):
        raw[..., 0:2] = _f16_bytes(_random_f16(rng, (N, nb), exp_lo, exp_hi))
    elif qtype == Q6_K:
        raw[..., 208:210] = _f16_bytes(_random_f16(rng, (N, nb), exp_lo, exp_hi))
    return raw.reshape(N, nb * BLOCK_BYTES[qtype])
