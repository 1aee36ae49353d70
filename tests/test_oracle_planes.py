"""Pins of the oracle's fp6 planes (R17): the Q4_K MMQ plane that mq_repack writes and
the fp6 section of the quantized activation plane.

Nothing here retypes the oracle's code: the E2M3 codes are checked against values
worked out by hand from the format (OCP FP6 E2M3: 1 sign, 2 exponent bits with bias 1,
3 mantissa bits); the bf16 hi/lo split against torch's own float -> bfloat16 rounding;
the byte layouts against a per-value brute force that places every bit with explicit
loops from fields read by the independent bit-by-bit decoder; and planted mistakes in
the oracle must fail those checks.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import bitwise_decode
from oracle import mq_oracle
from block_quantized_matmul_mq_amd import synth


# (value, code) pairs worked out by hand from the format: code = s ee mmm,
# value = m / 8 for e = 0, else 2^(e-1) (1 + m / 8)
HAND_E2M3 = [(0.0, 0b000000), (0.5, 0b000100), (1.0, 0b001000), (1.5, 0b001100), (2.0, 0b010000),
             (2.5, 0b010010), (3.5, 0b010110), (4.0, 0b011000), (4.5, 0b011001), (6.5, 0b011101),
             (7.5, 0b011111), (-0.5, 0b100100), (-4.0, 0b111000), (-3.5, 0b110110)]


@pytest.mark.parametrize("value,code", HAND_E2M3)
def test_e2m3_hand_worked_codes(value, code):
    assert oracle.e2m3_value(code) == value
    assert oracle.e2m3_code_of_half(int(2 * value)) == code


def test_e2m3_halves_are_exact_and_eight_is_not():
    # every multiple of 1/2 in [-7.5, 7.5] has exactly one code (0 as +0): the digits
    # h / 2 (h in -8..7) and l / 2, c / 2 (0..15) are exact; 8 itself is not a value,
    # which is why the digits are halved
    values = [oracle.e2m3_value(c) for c in range(64)]
    for k in range(-15, 16):
        hits = [c for c in range(64) if values[c] == k / 2 and not (k == 0 and c == 32)]
        assert hits == [oracle.e2m3_code_of_half(k)]
    assert 8.0 not in values and max(values) == 7.5


def test_fp6_record_bit_positions_by_hand():
    codes = np.zeros(32, dtype=np.uint8)
    codes[0] = 0b111111      # bits 0..5
    codes[1] = 0b000001      # bit 6
    codes[5] = 0b101010      # bits 30..35: bit 31, 33, 35 set
    codes[31] = 0b100000     # bit 191
    rec = oracle.fp6_records(codes)
    want = np.zeros(24, dtype=np.uint8)
    want[0] = 0x3F | 0x40
    want[3] = 0x80
    want[4] = 0x0A
    want[23] = 0x80
    assert np.array_equal(rec, want)


def test_bf16_hilo_matches_torch_rounding():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(4000).astype(np.float32) * np.float32(1e-3),
                        np.float32([0.0, 1.0, -2.5, 1.00390625, 1.005859375, 3e-38, 6e4])])
    hi, lo = oracle.bf16_hilo(x)

    def torch_bits(v):
        return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)

    assert np.array_equal(hi, torch_bits(x))
    hi_f = torch.from_numpy(hi.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(lo, torch_bits(x - hi_f))
    lo_f = torch.from_numpy(lo.view(np.int16)).view(torch.bfloat16).float().numpy()
    err = np.abs(x.astype(np.float64) - hi_f.astype(np.float64) - lo_f.astype(np.float64))
    normal = np.abs(x) >= 2.0 ** -100     # (lo of a value near the f32 minimum is subnormal)
    assert np.all(err[normal] <= 2.0 ** -16 * np.abs(x[normal].astype(np.float64)))


def _bf16_bits(v):
    return int(torch.tensor([float(v)], dtype=torch.float32).to(torch.bfloat16).view(torch.int16).item()) & 0xFFFF


def _bf16_split(v):
    """hi, lo bf16 bit patterns of an f32 value, through torch."""
    v = float(np.float32(v))
    hi = _bf16_bits(v)
    hi_f = float(torch.tensor([hi], dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float().item())
    lo = _bf16_bits(float(np.float32(v) - np.float32(hi_f)))
    return hi, lo


def _put_le(buf, off, word):
    for k in range(4):
        buf[off + k] = (word >> (8 * k)) & 0xFF


def _put_record(buf, off, codes6, first, count):
    """Bytes first .. first + count - 1 of the 24-byte record of 32 6-bit codes, placed bit
    by bit at buf[off ..]."""
    for byte in range(first, first + count):
        v = 0
        for bit in range(8):
            pos = 8 * byte + bit
            v |= ((int(codes6[pos // 6]) >> (pos % 6)) & 1) << bit
        buf[off + byte - first] = v


def brute_force_plane(raw, N, K):
    Np = -(-N // 256) * 256
    T = K // 64
    out = np.zeros(T * 80 * Np, dtype=np.uint8)
    blocks = raw.reshape(N, K // 256, 144)
    for n in range(N):
        for sb in range(K // 256):
            d, dmin, scales, mins, codes = bitwise_decode.q4_k_block_fields(blocks[n, sb])
            for j in range(8):
                b = 8 * sb + j
                t, u = divmod(b, 2)
                slab = t * 80 * Np
                c6 = [next(c for c in range(64) if oracle.e2m3_value(c) == codes[32 * j + i] / 2.0)
                      for i in range(32)]
                _put_record(out, slab + 16 * (u * Np + n), c6, 0, 16)
                _put_record(out, slab + 32 * Np + 8 * (u * Np + n), c6, 16, 8)
                dh, dl = _bf16_split(np.float32(d) * np.float32(scales[j]))
                mh, ml = _bf16_split(-(np.float32(dmin) * np.float32(mins[j])))
                _put_le(out, slab + 48 * Np + 8 * (u * Np + n), dh | (dh << 16))
                _put_le(out, slab + 48 * Np + 8 * (u * Np + n) + 4, dl | (dl << 16))
                _put_le(out, slab + 64 * Np + 8 * (u * Np + n), mh | (ml << 16))
                _put_le(out, slab + 64 * Np + 8 * (u * Np + n) + 4, mh | (ml << 16))
    return out


def brute_force_act(X):
    q, d, S = oracle.quantize_act(X)
    M, K = X.shape
    KB, T = K // 32, -(-K // 64)
    Mp = -(-M // 128) * 128
    out = np.zeros(T * 128 * Mp, dtype=np.uint8)
    for m in range(M):
        for b in range(KB):
            t, u = divmod(b, 2)
            slab = t * 128 * Mp
            vals = [int(v) for v in q[m, 32 * b:32 * b + 32]]
            hs = [next(c for c in range(64) if oracle.e2m3_value(c) == (v // 16) / 2.0 and not (v // 16 == 0 and c))
                  for v in vals]
            ls = [next(c for c in range(64) if oracle.e2m3_value(c) == (v % 16) / 2.0 and not (v % 16 == 0 and c))
                  for v in vals]
            for g, c6 in enumerate((hs, ls)):
                sp = 2 * u + g
                _put_record(out, slab + 16 * (sp * Mp + m), c6, 0, 16)
                _put_record(out, slab + 64 * Mp + 8 * (sp * Mp + m), c6, 16, 8)
            xh, xl = _bf16_split(d[m, b])
            th, tl = _bf16_split(np.float32(d[m, b]) * np.float32(S[m, b]))
            _put_le(out, slab + 96 * Mp + 8 * (u * Mp + m), xh | (xl << 16))
            _put_le(out, slab + 96 * Mp + 8 * (u * Mp + m) + 4, xh | (xl << 16))
            _put_le(out, slab + 112 * Mp + 8 * (u * Mp + m), th | (th << 16))
            _put_le(out, slab + 112 * Mp + 8 * (u * Mp + m) + 4, tl | (tl << 16))
    return out


@pytest.mark.parametrize("N,K,kind", [(3, 256, "random"), (2, 512, "quantized")])
def test_q4_k_plane_matches_brute_force(N, K, kind):
    rng = np.random.default_rng(11 + N)
    raw = synth.random_blocks(oracle.Q4_K, N, K, rng) if kind == "random" else \
        synth.quantized_weight(oracle.Q4_K, N, K, 91, N)
    got = oracle.repack(raw, oracle.Q4_K, N, K)
    assert got.size == (K // 64) * 80 * 256
    assert np.array_equal(got, brute_force_plane(raw, N, K))


@pytest.mark.parametrize("M,K", [(3, 96), (2, 256)])
def test_act_f6_section_matches_brute_force(M, K):
    X = synth.activations(M, K, config_index=13, tensor_index=M)
    X[0, :32] = 0.0                         # a zero block
    X[-1, 5] = 40.0                         # an outlier: codes of +-127 in its block
    q, d, S = oracle.quantize_act(X)
    got = oracle.act_f6_section(q, d, S)
    assert got.size == -(-K // 64) * 128 * 128
    assert np.array_equal(got, brute_force_act(X))


def test_plane_codes_round_trip_to_the_gguf_codes():
    N, K = 5, 768
    rng = np.random.default_rng(7)
    raw = synth.random_blocks(oracle.Q4_K, N, K, rng)
    plane = oracle.q4_k_plane(raw, N, K).reshape(K // 64, 80 * 256)
    codes = oracle.q4_k_fields(raw, N, K)[4].reshape(N, K // 32, 32)
    for t in range(K // 64):
        for u in range(2):
            rec = np.concatenate([plane[t, 16 * 256 * u:16 * 256 * (u + 1)].reshape(256, 16),
                                  plane[t, 32 * 256 + 8 * 256 * u:32 * 256 + 8 * 256 * (u + 1)].reshape(256, 8)],
                                 axis=1)
            bits = np.unpackbits(rec, axis=1, bitorder="little").reshape(256, 32, 6)
            c6 = (bits * (1 << np.arange(6))).sum(axis=2)
            vals = np.vectorize(oracle.e2m3_value)(c6)
            assert np.array_equal(2 * vals[:N], codes[:, 2 * t + u])
            assert not vals[N:].any()


def test_planted_mistakes_fail(monkeypatch):
    N, K = 2, 256
    raw = synth.quantized_weight(oracle.Q4_K, N, K, 91, 5)
    X = synth.activations(2, K, config_index=13, tensor_index=9)
    q, d, S = oracle.quantize_act(X)
    want_w, want_a = brute_force_plane(raw, N, K), brute_force_act(X)
    # the record's value order reversed
    orig = mq_oracle.fp6_records
    monkeypatch.setattr(mq_oracle, "fp6_records", lambda c: orig(np.asarray(c)[..., ::-1]))
    assert not np.array_equal(oracle.q4_k_plane(raw, N, K), want_w)
    assert not np.array_equal(oracle.act_f6_section(q, d, S), want_a)
    monkeypatch.setattr(mq_oracle, "fp6_records", orig)
    # hi and lo swapped
    orig_split = mq_oracle.bf16_hilo
    monkeypatch.setattr(mq_oracle, "bf16_hilo", lambda x: orig_split(x)[::-1])
    assert not np.array_equal(oracle.q4_k_plane(raw, N, K), want_w)
    assert not np.array_equal(oracle.act_f6_section(q, d, S), want_a)
    monkeypatch.setattr(mq_oracle, "bf16_hilo", orig_split)
    # the h digit taken as a logical shift of the code byte
    orig_code = mq_oracle.e2m3_code_of_half
    monkeypatch.setattr(mq_oracle, "e2m3_code_of_half", lambda k: orig_code(k % 16))
    assert not np.array_equal(oracle.act_f6_section(q, d, S), want_a)
