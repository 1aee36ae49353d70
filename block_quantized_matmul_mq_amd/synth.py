"""Seeded synthetic inputs: f32 weights/activations and their GGUF block encodings.

This module makes the inputs that both the HIP library and the CPU checks
consume.  It holds none of the matmul's arithmetic (no decode, no dot
product, no activation quantizer); it only draws seeded f32 tensors and
packs them into the GGUF block byte layouts Q8_0 (34 B / 32 values),
Q4_K (144 B / 256) and Q6_K (210 B / 256).  Sizes follow "minfer CUDA
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

Seeds: numpy ``default_rng(SeedSequence([0, config_index, tensor_index]))``.
"""

import numpy as np

Q8_0 = 8
Q4_K = 12
Q6_K = 14

BLOCK_VALUES = {Q8_0: 32, Q4_K: 256, Q6_K: 256}
BLOCK_BYTES = {Q8_0: 34, Q4_K: 144, Q6_K: 210}

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


ENCODERS = {Q8_0: encode_q8_0, Q4_K: encode_q4_k, Q6_K: encode_q6_k}


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
    elif qtype == Q4_K:
        raw[..., 0:2] = _f16_bytes(_random_f16(rng, (N, nb), exp_lo, exp_hi))
        raw[..., 2:4] = _f16_bytes(_random_f16(rng, (N, nb), exp_lo, exp_hi))
    elif qtype == Q6_K:
        raw[..., 208:210] = _f16_bytes(_random_f16(rng, (N, nb), exp_lo, exp_hi))
    return raw.reshape(N, nb * BLOCK_BYTES[qtype])
