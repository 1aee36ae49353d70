"""Second, independent block decoder (TEST INFRASTRUCTURE ONLY).

It decodes ONE block at a time in plain Python, building every field bit by
bit from a table of (byte, bit) positions, and reads f16 through the standard
library's IEEE half codec (``struct`` format 'e').  It shares no code with
``mq_oracle`` so that a slip in either (a swapped nibble, a wrong scale index,
a shifted qh pair) shows up as a disagreement on random bytes.

The layouts it reads are the public GGUF ones (Q8_0 34 B, Q4_0 18 B, Q4_1
20 B, Q5_0 22 B, Q5_1 24 B per 32 values; Q4_K 144 B, Q5_K 176 B, Q6_K 210 B
per 256); only some sizes are on the pages ("minfer CUDA Backend Design", 2.3
Weight residency and registry; "GPU Safety (Metal + CUDA Backends)", 3. Audit
findings).  GGUF interop: parity unpinned.
"""

import struct


def _bit(block, byte_index, bit_index):
    return (block[byte_index] >> bit_index) & 1


def _field(block, positions):
    """Assemble an unsigned integer; positions[k] = (byte, bit) of result bit k."""
    value = 0
    for k, (byte_index, bit_index) in enumerate(positions):
        value |= _bit(block, byte_index, bit_index) << k
    return value


def _half(block, offset):
    return struct.unpack("<e", bytes(block[offset:offset + 2]))[0]


def decode_q8_0_block(block):
    """34 bytes -> 32 floats: d (f16) times each signed byte."""
    block = bytes(bytearray(int(b) for b in block))
    assert len(block) == 34
    d = _half(block, 0)
    out = []
    for i in range(32):
        u = _field(block, [(2 + i, k) for k in range(8)])
        s = u - 256 if u >= 128 else u
        out.append(d * s)
    return out


def _q4_k_scale_min_positions(j):
    """(byte, bit) tables for the 6-bit scale and min of sub-block j (scale bytes start at 4)."""
    base = 4
    if j < 4:
        sc = [(base + j, k) for k in range(6)]
        mn = [(base + j + 4, k) for k in range(6)]
    else:
        sc = [(base + j + 4, k) for k in range(4)] + [(base + j - 4, 6), (base + j - 4, 7)]
        mn = [(base + j + 4, 4 + k) for k in range(4)] + [(base + j, 6), (base + j, 7)]
    return sc, mn


def decode_q4_k_block(block):
    """144 bytes -> 256 floats."""
    block = bytes(bytearray(int(b) for b in block))
    assert len(block) == 144
    d = _half(block, 0)
    dmin = _half(block, 2)
    out = []
    for e in range(256):
        j = e // 32
        sc_pos, mn_pos = _q4_k_scale_min_positions(j)
        sc = _field(block, sc_pos)
        mn = _field(block, mn_pos)
        chunk, r = divmod(e, 64)
        byte_index = 16 + 32 * chunk + (r % 32)
        first_bit = 0 if r < 32 else 4
        code = _field(block, [(byte_index, first_bit + k) for k in range(4)])
        out.append(d * sc * code - dmin * mn)
    return out


def q4_k_block_fields(block):
    """144 bytes -> (d, dmin, [8 scales], [8 mins], [256 codes]) as plain Python numbers,
    every field read bit by bit (the codes as unsigned 4-bit integers)."""
    block = bytes(bytearray(int(b) for b in block))
    assert len(block) == 144
    scales, mins = [], []
    for j in range(8):
        sc_pos, mn_pos = _q4_k_scale_min_positions(j)
        scales.append(_field(block, sc_pos))
        mins.append(_field(block, mn_pos))
    codes = []
    for e in range(256):
        chunk, r = divmod(e, 64)
        byte_index = 16 + 32 * chunk + (r % 32)
        first_bit = 0 if r < 32 else 4
        codes.append(_field(block, [(byte_index, first_bit + k) for k in range(4)]))
    return _half(block, 0), _half(block, 2), scales, mins, codes


def decode_q6_k_block(block):
    """210 bytes -> 256 floats."""
    block = bytes(bytearray(int(b) for b in block))
    assert len(block) == 210
    d = _half(block, 208)
    out = []
    for e in range(256):
        h, r = divmod(e, 128)
        t, l = divmod(r, 32)
        ql_byte = 64 * h + l + (32 if t in (1, 3) else 0)
        ql_first = 4 if t >= 2 else 0
        qh_byte = 128 + 32 * h + l
        positions = [(ql_byte, ql_first + k) for k in range(4)]
        positions += [(qh_byte, 2 * t), (qh_byte, 2 * t + 1)]
        code = _field(block, positions)
        su = block[192 + e // 16]
        scale = su - 256 if su >= 128 else su
        out.append(d * scale * (code - 32))
    return out


def _legacy(block, nbytes, has_min, has_high, offset):
    """Shared walk of the 32-value types: f16 d, [f16 m], [qh: 32 bits], 16 nibble bytes."""
    block = bytes(bytearray(int(b) for b in block))
    assert len(block) == nbytes
    d = _half(block, 0)
    m = _half(block, 2) if has_min else 0.0
    qh_at = 4 if has_min else 2
    qs_at = qh_at + (4 if has_high else 0)
    out = []
    for i in range(32):
        byte_index = qs_at + (i % 16)
        first_bit = 0 if i < 16 else 4
        positions = [(byte_index, first_bit + k) for k in range(4)]
        if has_high:
            positions.append((qh_at + i // 8, i % 8))
        code = _field(block, positions)
        out.append(d * (code - offset) + m)
    return out


def decode_q4_0_block(block):
    """18 bytes -> 32 floats: d * (code - 8)."""
    return _legacy(block, 18, False, False, 8)


def decode_q4_1_block(block):
    """20 bytes -> 32 floats: d * code + m."""
    return _legacy(block, 20, True, False, 0)


def decode_q5_0_block(block):
    """22 bytes -> 32 floats: d * (code - 16), 5-bit codes."""
    return _legacy(block, 22, False, True, 16)


def decode_q5_1_block(block):
    """24 bytes -> 32 floats: d * code + m, 5-bit codes."""
    return _legacy(block, 24, True, True, 0)


def decode_q5_k_block(block):
    """176 bytes -> 256 floats (Q4_K header, 32 bytes qh at 16, nibbles at 48)."""
    block = bytes(bytearray(int(b) for b in block))
    assert len(block) == 176
    d = _half(block, 0)
    dmin = _half(block, 2)
    out = []
    for e in range(256):
        j = e // 32
        sc_pos, mn_pos = _q4_k_scale_min_positions(j)
        sc = _field(block, sc_pos)
        mn = _field(block, mn_pos)
        chunk, r = divmod(e, 64)
        byte_index = 48 + 32 * chunk + (r % 32)
        first_bit = 0 if r < 32 else 4
        positions = [(byte_index, first_bit + k) for k in range(4)] + [(16 + e % 32, j)]
        code = _field(block, positions)
        out.append(d * sc * code - dmin * mn)
    return out
