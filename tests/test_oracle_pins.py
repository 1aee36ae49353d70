"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test fixes the oracle to a hand-worked block, a closed form, an exact
rational brute force, a library routine or an invariant.  The mutation tests
at the bottom plant plausible mistakes in the oracle (on the CPU) and show
that some pin here fails for each.
"""

import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import bitwise_decode, mq_oracle
from block_quantized_matmul_mq_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
Q8_0, Q4_K, Q6_K = oracle.Q8_0, oracle.Q4_K, oracle.Q6_K


def f16_le(value):
    return list(struct.pack("<e", value))


# --------------------------------------------------------------------------
# Helpers that build blocks by hand (a third statement of the layout, written
# from the field description only) and closed-form expected values.
# --------------------------------------------------------------------------

def handmade_q8_0(d, codes):
    assert len(codes) == 32
    return bytes(f16_le(d) + [c & 0xFF for c in codes])


def handmade_q4_k(d, dmin, sc, mn, code_of):
    """code_of(e) -> 4-bit code of value e."""
    scales = [0] * 12
    for j in range(8):
        if j < 4:
            scales[j] |= sc[j]
            scales[j + 4] |= mn[j]
        else:
            scales[j + 4] |= (sc[j] & 0xF) | ((mn[j] & 0xF) << 4)
            scales[j - 4] |= (sc[j] >> 4) << 6
            scales[j] |= (mn[j] >> 4) << 6
    qs = [0] * 128
    for e in range(256):
        chunk, r = divmod(e, 64)
        if r < 32:
            qs[32 * chunk + r] |= code_of(e)
        else:
            qs[32 * chunk + r - 32] |= code_of(e) << 4
    return bytes(f16_le(d) + f16_le(dmin) + scales + qs)


def handmade_q6_k(d, scales, code_of):
    ql = [0] * 128
    qh = [0] * 64
    for e in range(256):
        c = code_of(e)
        h, r = divmod(e, 128)
        t, l = divmod(r, 32)
        ql[64 * h + l + 32 * (t % 2)] |= (c & 0xF) << (4 * (t // 2))
        qh[32 * h + l] |= (c >> 4) << (2 * t)
    return bytes(ql + qh + [s & 0xFF for s in scales] + f16_le(d))


def as_raw(blocks):
    return np.frombuffer(b"".join(blocks), dtype=np.uint8)


# --------------------------------------------------------------------------
# Sizes and the f16 codec
# --------------------------------------------------------------------------

def read_sizes():
    sizes = {}
    with open(os.path.join(GOLDEN, "block_sizes.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                name, vals, nbytes = line.split()
                sizes[name] = (int(vals), int(nbytes))
    return sizes


def test_block_sizes_match_the_pages():
    sizes = read_sizes()
    assert (oracle.BLOCK_VALUES[Q8_0], oracle.BLOCK_BYTES[Q8_0]) == sizes["Q8_0"]
    assert (oracle.BLOCK_VALUES[Q4_K], oracle.BLOCK_BYTES[Q4_K]) == sizes["Q4_K"]
    assert oracle.BLOCK_BYTES[Q6_K] < sizes["Q6_K_PADDED_SLOT"][1]
    assert oracle.BLOCK_BYTES[Q6_K] == 128 + 64 + 16 + 2
    # the q4_0 ratio equals q4_K's: a size check alone cannot tell them apart
    assert Fraction(*sizes["Q4_0"][::-1]) == Fraction(*sizes["Q4_K"][::-1])
    assert oracle.row_bytes(Q4_K, 3584) == 14 * 144
    assert oracle.row_bytes(Q8_0, 896) == 28 * 34


def test_repacked_slots_follow_the_pages_and_their_alignment():
    sizes = read_sizes()
    slot6, off6 = oracle.REPACK_SLOT[Q6_K]
    # the page's Q6_K slot, and what it is for: every slot starts 16-byte aligned
    assert slot6 == sizes["Q6_K_PADDED_SLOT"][1] and slot6 % 16 == 0
    assert off6 + oracle.BLOCK_BYTES[Q6_K] <= slot6
    slot8, off8 = oracle.REPACK_SLOT[Q8_0]
    # the Q8_0 codes follow the 2-byte scale: they must start 4-byte aligned
    assert slot8 % 4 == 0 and (off8 + 2) % 4 == 0 and off8 + oracle.BLOCK_BYTES[Q8_0] <= slot8


@pytest.mark.parametrize("qtype", [Q8_0, Q6_K], ids=["q8_0", "q6_K"])
def test_repack_brute_force_and_round_trip(qtype):
    rng = np.random.default_rng(qtype)
    bv, bb = oracle.BLOCK_VALUES[qtype], oracle.BLOCK_BYTES[qtype]
    N, nb = 3, 2
    K = nb * bv
    raw = rng.integers(0, 256, N * nb * bb, dtype=np.uint8)
    rep = oracle.repack(raw, qtype, N, K)
    slot, off = oracle.REPACK_SLOT[qtype]
    assert rep.size == N * nb * slot
    for n in range(N):              # byte by byte: slot (n, b) holds block (n, b) at off, zeros elsewhere
        for b in range(nb):
            for j in range(slot):
                want = raw[(n * nb + b) * bb + j - off] if off <= j < off + bb else 0
                assert rep[(n * nb + b) * slot + j] == want
    assert np.array_equal(oracle.unpack_repacked(rep, qtype, N, K), raw)
    bad = rep.copy()
    bad[slot - 1 if off == 0 else 0] = 1     # a padding byte
    with pytest.raises(ValueError):
        oracle.unpack_repacked(bad, qtype, N, K)
    with pytest.raises(ValueError):
        oracle.unpack_repacked(rep[:-1], qtype, N, K)


def test_payload_length_must_be_exact():
    raw = np.zeros(2 * 144, dtype=np.uint8)
    oracle.decode(raw, Q4_K, 2, 256)
    for bad in (raw[:-1], np.zeros(2 * 144 + 1, dtype=np.uint8)):
        with pytest.raises(ValueError):
            oracle.decode(bad, Q4_K, 2, 256)


def test_f16_decoder_matches_ieee_library_on_every_finite_pattern():
    bits = np.arange(65536, dtype=np.uint32)
    finite = ((bits >> 10) & 0x1F) != 0x1F
    bits = bits[finite]
    lo = (bits & 0xFF).astype(np.uint8)
    hi = (bits >> 8).astype(np.uint8)
    ours = oracle.f16_bits_to_f64(lo, hi)
    lib = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    assert np.array_equal(ours, lib)
    assert oracle.f16_bits_to_f64(np.array([0x00], np.uint8), np.array([0x3C], np.uint8))[0] == 1.0
    assert oracle.f16_bits_to_f64(np.array([0x01], np.uint8), np.array([0x00], np.uint8))[0] == 2.0 ** -24


# --------------------------------------------------------------------------
# Hand-worked blocks with closed-form values
# --------------------------------------------------------------------------

@pytest.mark.parametrize("qtype,K", [(Q8_0, 32), (Q4_K, 256), (Q6_K, 256)])
def test_all_zero_block_decodes_to_zero(qtype, K):
    raw = np.zeros(oracle.BLOCK_BYTES[qtype], dtype=np.uint8)
    w = oracle.decode(raw, qtype, 1, K)
    if qtype == Q6_K:
        # code 0 means -32 but the scale and d are 0
        assert np.all(w == 0)
    else:
        assert np.all(w == 0)


def test_q8_0_unit_scale_gives_the_codes():
    codes = list(range(-128, 128))
    blocks = [handmade_q8_0(1.0, codes[32 * i:32 * i + 32]) for i in range(8)]
    w = oracle.decode(as_raw(blocks), Q8_0, 1, 256)
    assert np.array_equal(w.reshape(-1), np.array(codes, dtype=np.float64))
    blocks = [handmade_q8_0(-0.375, codes[32 * i:32 * i + 32]) for i in range(8)]
    w = oracle.decode(as_raw(blocks), Q8_0, 1, 256)
    assert np.array_equal(w.reshape(-1), -0.375 * np.array(codes, dtype=np.float64))


def q4_k_handworked():
    d, dmin = 1.0, 0.5
    sc = [40 + j for j in range(8)]          # j >= 4 needs the high 2 bits (44..47)
    mn = [17 + 2 * j for j in range(8)]      # 25..31 for j >= 4
    code_of = lambda e: (e + e // 32) % 16   # low and high nibble of a byte differ
    block = handmade_q4_k(d, dmin, sc, mn, code_of)
    expect = [d * sc[e // 32] * code_of(e) - dmin * mn[e // 32] for e in range(256)]
    return block, np.array(expect)


def test_q4_k_handworked_block():
    block, expect = q4_k_handworked()
    assert block[4:16].hex() == "a8a9aaab515355579cbddeff"  # by hand: 6-bit packing
    w = oracle.decode(as_raw([block]), Q4_K, 1, 256)
    assert np.array_equal(w.reshape(-1), expect)


def q6_k_handworked():
    d = 0.125
    scales = [(-1) ** g * (7 * g + 3) for g in range(16)]   # negative sub-scales included
    scales[15] = -128
    code_of = lambda e: (5 * e + e // 16) % 64
    block = handmade_q6_k(d, scales, code_of)
    expect = [d * scales[e // 16] * (code_of(e) - 32) for e in range(256)]
    return block, np.array(expect)


def test_q6_k_handworked_block():
    block, expect = q6_k_handworked()
    w = oracle.decode(as_raw([block]), Q6_K, 1, 256)
    assert np.array_equal(w.reshape(-1), expect)


def test_q6_k_every_code_pattern():
    # each of the 64 codes at every value position, via a rotating pattern
    for shift in range(0, 64, 7):
        code_of = lambda e, s=shift: (e + s) % 64
        block = handmade_q6_k(1.0, [1] * 16, code_of)
        w = oracle.decode(as_raw([block]), Q6_K, 1, 256).reshape(-1)
        assert np.array_equal(w, np.array([code_of(e) - 32 for e in range(256)], dtype=np.float64))


# --------------------------------------------------------------------------
# Independent decoder cross-check
# --------------------------------------------------------------------------

BITWISE = {Q8_0: bitwise_decode.decode_q8_0_block,
           Q4_K: bitwise_decode.decode_q4_k_block,
           Q6_K: bitwise_decode.decode_q6_k_block}


@pytest.mark.parametrize("qtype", [Q8_0, Q4_K, Q6_K])
def test_vectorised_decoder_matches_bitwise_decoder_on_random_bytes(qtype):
    rng = np.random.default_rng(7 + qtype)
    N, K = 6, 512
    raw = synth.random_blocks(qtype, N, K, rng)
    w = oracle.decode(raw, qtype, N, K).reshape(-1)
    alt = np.concatenate([BITWISE[qtype](blk) for blk in raw.reshape(-1, oracle.BLOCK_BYTES[qtype])])
    assert np.array_equal(w, alt)


# --------------------------------------------------------------------------
# Weight generators: round trip bounds and invariants
# --------------------------------------------------------------------------

def _roundtrip_bound(qtype, raw, N, K):
    if qtype == Q8_0:
        d, _ = oracle.q8_0_fields(raw, N, K)
        return np.repeat(np.abs(d), 32, axis=-1).reshape(N, K) / 2
    if qtype == Q4_K:
        d, _, sc, _, _ = oracle.q4_k_fields(raw, N, K)
        return np.repeat(np.abs(d)[..., None] * sc, 32, axis=-1).reshape(N, K) / 2
    d, s, _ = oracle.q6_k_fields(raw, N, K)
    return np.repeat(np.abs(d[..., None] * s), 16, axis=-1).reshape(N, K) / 2


@pytest.mark.parametrize("qtype", [Q8_0, Q4_K, Q6_K])
def test_generator_roundtrip_bound(qtype):
    rng = np.random.default_rng(11)
    N, K = 64, 1024
    W = synth.normal_f32(rng, (N, K), 0.02)
    W[0, :256] *= 40.0             # wide-range row
    W[1, :32] = 0.0                # a zero sub-block inside a live block
    raw = synth.ENCODERS[qtype](W)
    deq = oracle.decode(raw, qtype, N, K)
    bound = _roundtrip_bound(qtype, raw, N, K)
    err = np.abs(deq - W.astype(np.float64))
    assert np.all(err <= bound * (1 + 1e-6) + 1e-30)


@pytest.mark.parametrize("qtype", [Q8_0, Q4_K, Q6_K])
def test_generator_zero_input_gives_zero_blocks(qtype):
    raw = synth.ENCODERS[qtype](np.zeros((3, 512), dtype=np.float32))
    if qtype == Q6_K:
        # codes are 32 (value 0) with zero scales; the ql/qh bytes hold code 32
        assert np.all(oracle.decode(raw, qtype, 3, 512) == 0)
        assert np.all(raw.reshape(-1, 210)[:, 192:] == 0)
    else:
        assert np.all(raw == 0)


@pytest.mark.parametrize("qtype", [Q8_0, Q6_K])
def test_generator_sign_symmetry(qtype):
    rng = np.random.default_rng(12)
    W = synth.normal_f32(rng, (16, 512), 0.02)
    a = oracle.decode(synth.ENCODERS[qtype](W), qtype, 16, 512)
    b = oracle.decode(synth.ENCODERS[qtype](-W), qtype, 16, 512)
    assert np.array_equal(a, -b)


@pytest.mark.parametrize("qtype", [Q8_0, Q4_K, Q6_K])
def test_generator_power_of_two_scaling(qtype):
    rng = np.random.default_rng(13)
    W = synth.normal_f32(rng, (16, 512), 0.02) * np.float32(16.0)   # keeps f16 scales normal
    a = oracle.decode(synth.ENCODERS[qtype](W), qtype, 16, 512)
    b = oracle.decode(synth.ENCODERS[qtype](W * np.float32(4.0)), qtype, 16, 512)
    assert np.array_equal(4.0 * a, b)


def test_q8_0_generator_is_idempotent():
    rng = np.random.default_rng(14)
    W = synth.normal_f32(rng, (8, 256), 0.02)
    raw = synth.encode_q8_0(W)
    again = synth.encode_q8_0(oracle.decode(raw, Q8_0, 8, 256).astype(np.float32))
    assert np.array_equal(raw, again)


# --------------------------------------------------------------------------
# Activation quantizer
# --------------------------------------------------------------------------

def read_rounding_rules(name="q8_rounding_rules.txt"):
    xs, qs = [], []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                x, q = line.split()
                xs.append(float(x))
                qs.append(int(q))
    return xs, qs


@pytest.mark.parametrize("name,scale", [("q8_rounding_rules.txt", 1.0),
                                        ("q8_rounding_rules_scale7.txt", 7.0)])
def test_act_quantizer_worked_ties(name, scale):
    xs, qs = read_rounding_rules(name)
    block = np.zeros((1, 32), dtype=np.float32)
    block[0, :len(xs)] = xs
    q, d, S = oracle.quantize_act(block)
    assert d[0, 0] == np.float32(scale)
    assert list(q[0, :len(xs)]) == qs
    assert S[0, 0] == sum(qs)


def test_act_quantizer_zero_block():
    X = np.zeros((2, 64), dtype=np.float32)
    X[1, 32:] = 3.0
    q, d, S = oracle.quantize_act(X)
    assert d[0, 0] == 0 and d[0, 1] == 0 and d[1, 0] == 0
    assert np.all(q[0] == 0) and np.all(q[1, :32] == 0)
    assert np.all(q[1, 32:] == 127) and S[1, 1] == 127 * 32


def test_act_quantizer_sign_symmetry_and_power_of_two():
    rng = np.random.default_rng(21)
    X = synth.normal_f32(rng, (8, 1024))
    q, d, S = oracle.quantize_act(X)
    qn, dn, Sn = oracle.quantize_act(-X)
    assert np.array_equal(q, -qn) and np.array_equal(d, dn) and np.array_equal(S, -Sn)
    for k in (-20, -3, 5, 30):
        qk, dk, _ = oracle.quantize_act(X * np.float32(2.0 ** k))
        assert np.array_equal(qk, q)
        assert np.array_equal(dk, d * np.float32(2.0 ** k))


def _round_fraction_to_f32(fr):
    """Correctly rounded (ties to even) f32 value of a positive or negative Fraction."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)                    # subnormal range keeps the same spacing
    scaled = a / Fraction(2) ** (e - 23)
    m = _round_half_even(scaled)
    return sign * Fraction(m) * Fraction(2) ** (e - 23)


def _round_half_even(fr):
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def test_act_quantizer_brute_force_exact_rationals():
    rng = np.random.default_rng(22)
    X = synth.normal_f32(rng, (3, 96)) * np.float32(3.0)
    X[0, 5] = X[0, 7] = 0.0
    X[2, 32:64] = np.float32(0.5) * np.arange(32, dtype=np.float32) - np.float32(8.0)  # exact ties
    q, d, S = oracle.quantize_act(X)
    for m in range(X.shape[0]):
        for b in range(X.shape[1] // 32):
            vals = [Fraction(float(v)) for v in X[m, 32 * b:32 * b + 32]]
            amax = max(abs(v) for v in vals)
            dd = _round_fraction_to_f32(amax / 127)
            assert Fraction(float(d[m, b])) == dd
            for i, v in enumerate(vals):
                expect = 0 if dd == 0 else _round_half_even(_round_fraction_to_f32(v / dd))
                expect = max(-127, min(127, expect))
                assert q[m, 32 * b + i] == expect
            assert S[m, b] == sum(int(c) for c in q[m, 32 * b:32 * b + 32])


# --------------------------------------------------------------------------
# GEMV and MMQ
# --------------------------------------------------------------------------

def _exact_gemv(raw, qtype, x, N, K):
    bb = oracle.BLOCK_BYTES[qtype]
    per_row = K // oracle.BLOCK_VALUES[qtype]
    flat = raw.reshape(-1, bb)
    out = []
    for n in range(N):
        w = []
        for blk in flat[n * per_row:(n + 1) * per_row]:
            w.extend(BITWISE[qtype](blk))
        out.append(sum(Fraction(a) * Fraction(float(b)) for a, b in zip(w, x)))
    return out


@pytest.mark.parametrize("qtype", [Q8_0, Q4_K, Q6_K])
def test_gemv_brute_force_4x256_exact(qtype):
    rng = np.random.default_rng(31 + qtype)
    N, K = 4, 256
    raw = synth.random_blocks(qtype, N, K, rng)
    x = synth.normal_f32(rng, (K,))
    y = oracle.gemv(raw, qtype, x, N, K)
    exact = _exact_gemv(raw, qtype, x, N, K)
    w = oracle.decode(raw, qtype, N, K)
    for n in range(N):
        scale = np.linalg.norm(w[n]) * np.linalg.norm(x.astype(np.float64))
        assert abs(Fraction(float(y[n])) - exact[n]) <= Fraction(1e-15) * Fraction(scale)


def test_gemv_closed_forms():
    K = 512
    blocks = [handmade_q8_0(0.25, [5] * 32) for _ in range(K // 32)]
    assert np.all(oracle.gemv(as_raw(blocks), Q8_0, np.ones(K, np.float32), 1, K) == 1.25 * K)
    blk = handmade_q4_k(1.0, 0.5, [2] * 8, [1] * 8, lambda e: 3)
    assert np.all(oracle.gemv(as_raw([blk, blk]), Q4_K, np.ones(K, np.float32), 1, K) == 5.5 * K)
    blk = handmade_q6_k(0.5, [-3] * 16, lambda e: 40)
    assert np.all(oracle.gemv(as_raw([blk, blk]), Q6_K, np.ones(K, np.float32), 1, K) == -12.0 * K)


@pytest.mark.parametrize("qtype", [Q8_0, Q4_K, Q6_K])
def test_gemv_linearity(qtype):
    rng = np.random.default_rng(41)
    N, K = 8, 512
    raw = synth.random_blocks(qtype, N, K, rng)
    x1 = rng.integers(-1000, 1000, K).astype(np.float32)
    x2 = rng.integers(-1000, 1000, K).astype(np.float32)
    y = oracle.gemv(raw, qtype, 3 * x1 - 2 * x2, N, K)
    ylin = 3 * oracle.gemv(raw, qtype, x1, N, K) - 2 * oracle.gemv(raw, qtype, x2, N, K)
    scale = np.abs(oracle.decode(raw, qtype, N, K)).sum(axis=1) * 5000
    assert np.all(np.abs(y - ylin) <= 1e-12 * scale)


def test_mmq_reduces_to_integer_matmul():
    # Q8_0 weights with d = 1 and integer activations whose every block has
    # amax 127 make every scale exactly 1: the product is a plain int matmul.
    rng = np.random.default_rng(51)
    M, N, K = 5, 7, 256
    Wi = rng.integers(-127, 128, (N, K))
    Xi = rng.integers(-127, 128, (M, K))
    Xi.reshape(M, K // 32, 32)[..., 0] = 127
    blocks = [handmade_q8_0(1.0, list(Wi[n, 32 * b:32 * b + 32])) for n in range(N) for b in range(K // 32)]
    raw = as_raw(blocks)
    q, d, S = oracle.quantize_act(Xi.astype(np.float32))
    assert np.all(d == 1.0) and np.array_equal(q, Xi)
    Y = oracle.mmq(raw, Q8_0, q, d, N, K)
    assert np.array_equal(Y, (Xi @ Wi.T).astype(np.float64))
    D = oracle.block_dots(raw, Q8_0, q, N, K)
    assert np.array_equal(D.sum(axis=-1), Xi @ Wi.T)


@pytest.mark.parametrize("qtype", [Q8_0, Q4_K, Q6_K])
def test_mmq_equals_block_dot_form(qtype):
    rng = np.random.default_rng(61 + qtype)
    M, N, K = 6, 10, 512
    raw = synth.random_blocks(qtype, N, K, rng)
    X = synth.normal_f32(rng, (M, K))
    q, d, S = oracle.quantize_act(X)
    a = oracle.mmq(raw, qtype, q, d, N, K)
    b = oracle.mmq_from_block_dots(raw, qtype, q, d, S, N, K)
    w = oracle.decode(raw, qtype, N, K)
    xh = (q.reshape(M, -1, 32) * d[..., None].astype(np.float64)).reshape(M, K)
    scale = np.outer(np.linalg.norm(xh, axis=1), np.linalg.norm(w, axis=1))
    assert np.all(np.abs(a - b) <= 1e-14 * scale)


@pytest.mark.parametrize("qtype", [Q8_0, Q4_K, Q6_K])
def test_block_dots_brute_force(qtype):
    rng = np.random.default_rng(71 + qtype)
    M, N, K = 2, 3, 256
    raw = synth.random_blocks(qtype, N, K, rng)
    q, _, _ = oracle.quantize_act(synth.normal_f32(rng, (M, K)))
    D = oracle.block_dots(raw, qtype, q, N, K)
    bb = oracle.BLOCK_BYTES[qtype]
    grp = 16 if qtype == Q6_K else 32
    for n in range(N):
        codes = []
        for blk in raw.reshape(N, -1)[n].reshape(-1, bb):
            blk = blk.tobytes()
            # codes recovered through the bitwise decoder with a unit scale patched in
            if qtype == Q8_0:
                vals = bitwise_decode.decode_q8_0_block(f16_le(1.0) + list(blk[2:]))
            elif qtype == Q4_K:
                patched = f16_le(1.0) + f16_le(0.0) + [1, 1, 1, 1, 0, 0, 0, 0, 1, 1, 1, 1] + list(blk[16:])
                vals = bitwise_decode.decode_q4_k_block(patched)
            else:
                patched = list(blk[:192]) + [1] * 16 + f16_le(1.0)
                vals = bitwise_decode.decode_q6_k_block(patched)
            codes.extend(int(v) for v in vals)
        for m in range(M):
            for g in range(K // grp):
                expect = sum(codes[grp * g + i] * int(q[m, grp * g + i]) for i in range(grp))
                assert D[m, n, g] == expect


@pytest.mark.parametrize("qtype", [Q8_0, Q4_K, Q6_K])
def test_gemv_vs_mmq_cross_bound(qtype):
    rng = np.random.default_rng(81)
    N, K = 12, 1024
    raw = synth.random_blocks(qtype, N, K, rng)
    x = synth.normal_f32(rng, (1, K))
    q, d, _ = oracle.quantize_act(x)
    y2 = oracle.gemv(raw, qtype, x[0], N, K)
    y5 = oracle.mmq(raw, qtype, q, d, N, K)[0]
    w = np.abs(oracle.decode(raw, qtype, N, K)).reshape(N, K // 32, 32).sum(axis=-1)
    bound = (w * (d[0].astype(np.float64) / 2)).sum(axis=-1)
    assert np.all(np.abs(y2 - y5) <= bound * (1 + 1e-9))
    assert np.any(np.abs(y2 - y5) > 0)


# --------------------------------------------------------------------------
# Planted mistakes: each mutant of the oracle must fail at least one pin.
# --------------------------------------------------------------------------

def _mutant_fields(original, transform):
    def fields(raw, N, K):
        return transform(*original(raw, N, K))
    return fields


def _swap_q4_nibbles(d, dmin, sc, mn, codes):
    c = codes.copy().reshape(codes.shape[:-1] + (4, 2, 32))
    return d, dmin, sc, mn, c[..., ::-1, :].reshape(codes.shape)


def _shift_q4_scale_index(d, dmin, sc, mn, codes):
    return d, dmin, np.roll(sc, 1, axis=-1), mn, codes


def _drop_q4_min(d, dmin, sc, mn, codes):
    return d, dmin * 0, sc, mn, codes


def _q4_high_bits_from_wrong_byte(d, dmin, sc, mn, codes):
    mn = mn.copy()
    mn[..., 4:] = mn[..., 4:] & 15
    return d, dmin, sc, mn, codes


def _q6_unsigned_scales(d, scales, codes):
    return d, scales & 0xFF, codes


def _q6_qh_shift_halved(d, scales, codes):
    c = codes.copy()
    c[..., 32:64] = (c[..., 32:64] & 15) | ((c[..., 64:96] >> 4) << 4)
    return d, scales, c


def _q8_unsigned_codes(d, q):
    return d, q & 0xFF


MUTANTS = [
    ("q4_k_fields", _swap_q4_nibbles),
    ("q4_k_fields", _shift_q4_scale_index),
    ("q4_k_fields", _drop_q4_min),
    ("q4_k_fields", _q4_high_bits_from_wrong_byte),
    ("q6_k_fields", _q6_unsigned_scales),
    ("q6_k_fields", _q6_qh_shift_halved),
    ("q8_0_fields", _q8_unsigned_codes),
]

DECODER_PINS = [
    test_q4_k_handworked_block,
    test_q6_k_handworked_block,
    test_q8_0_unit_scale_gives_the_codes,
]


@pytest.mark.parametrize("name,transform", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_planted_decoder_mistakes_are_caught(monkeypatch, name, transform):
    original = getattr(mq_oracle, name)
    monkeypatch.setattr(mq_oracle, name, _mutant_fields(original, transform))
    failures = 0
    for pin in DECODER_PINS:
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1


def _quantize_act_times_reciprocal(X):
    X = np.asarray(X, dtype=np.float32)
    M, K = X.shape
    xb = X.reshape(M, K // 32, 32)
    d = (np.max(np.abs(xb), axis=-1) / np.float32(127)).astype(np.float32)
    inv = np.where(d > 0, np.float32(1) / np.where(d > 0, d, 1), 0).astype(np.float32)
    q = np.clip(np.rint(xb * inv[..., None]), -127, 127).astype(np.int8)
    return q.reshape(M, K), d, q.astype(np.int32).sum(-1)


def _quantize_act_half_away(X):
    X = np.asarray(X, dtype=np.float32)
    M, K = X.shape
    xb = X.reshape(M, K // 32, 32)
    d = (np.max(np.abs(xb), axis=-1) / np.float32(127)).astype(np.float32)
    r = xb / np.where(d > 0, d, 1)[..., None]
    q = np.clip(np.sign(r) * np.floor(np.abs(r) + 0.5), -127, 127).astype(np.int8)
    return q.reshape(M, K), d, q.astype(np.int32).sum(-1)


def _quantize_act_amax_126(X):
    X = np.asarray(X, dtype=np.float32)
    M, K = X.shape
    xb = X.reshape(M, K // 32, 32)
    d = (np.max(np.abs(xb), axis=-1) / np.float32(126)).astype(np.float32)
    q = np.clip(np.rint(xb / np.where(d > 0, d, 1)[..., None]), -127, 127).astype(np.int8)
    return q.reshape(M, K), d, q.astype(np.int32).sum(-1)


@pytest.mark.parametrize("mutant", [_quantize_act_times_reciprocal, _quantize_act_half_away,
                                    _quantize_act_amax_126])
def test_planted_quantizer_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(oracle, "quantize_act", mutant)
    failures = 0
    pins = [lambda: test_act_quantizer_worked_ties("q8_rounding_rules.txt", 1.0),
            lambda: test_act_quantizer_worked_ties("q8_rounding_rules_scale7.txt", 7.0),
            test_act_quantizer_brute_force_exact_rationals]
    for pin in pins:
        try:
            pin()
        except AssertionError:
            failures += 1
    assert failures >= 1
