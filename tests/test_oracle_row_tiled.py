"""Pins of the oracle's Q4_K row-tiled layout (reading R18): rows in groups of
R = min(16, ceil(N / 256)), a group's super-block s blocks stored one after another
in row order, then s + 1; the last group filled with zero rows.

The layout function is a reshape and a transpose; here it is checked against a
block-by-block construction that walks the stated order, against an inverse
written as a loop over the groups, and against the group sizes and byte counts the
layout states."""

import numpy as np
import pytest

import oracle
from block_quantized_matmul_mq_amd import synth


def built_block_by_block(raw, N, K):
    # walk the stated order: groups, then super-blocks, then the group's rows
    SB = K // 256
    rows = raw.reshape(N, SB, 144)
    R = oracle.row_tile_rows(N)
    out = []
    for g0 in range(0, N, R):
        for s in range(SB):
            for n in range(g0, g0 + R):
                out.append(rows[n, s] if n < N else np.zeros(144, dtype=np.uint8))
    return np.concatenate(out)


def test_rows_per_group():
    # at most 256 groups for up to 4096 rows, 16-row groups beyond
    got = [oracle.row_tile_rows(n) for n in (1, 255, 256, 257, 512, 513, 3584, 4095, 4096, 4097, 18944, 10 ** 6)]
    assert got == [1, 1, 1, 2, 2, 3, 14, 16, 16, 16, 16, 16]


@pytest.mark.parametrize("N,K", [(3, 17 * 256), (300, 17 * 256), (513, 18 * 256), (700, 20 * 256)])
def test_matches_block_by_block_construction_and_inverts(N, K):
    raw = synth.random_blocks(oracle.Q4_K, N, K, np.random.default_rng(N)).reshape(-1)
    tiled = oracle.q4_k_row_tiled(raw, N, K)
    assert np.array_equal(tiled, built_block_by_block(raw, N, K))
    R = oracle.row_tile_rows(N)
    assert tiled.size == -(-N // R) * R * (K // 256) * 144
    assert np.array_equal(oracle.unpack_q4_k_row_tiled(tiled, N, K), raw)


def test_group_of_the_7b_ffn_down_shape():
    # 3584 x 18944: 14-row groups, no filler; group g's super-block s is the 2016
    # contiguous bytes at (74 g + s) * 2016 and holds rows 14 g .. 14 g + 13
    N, K = 3584, 18944
    raw = synth.random_blocks(oracle.Q4_K, N, K, np.random.default_rng(1)).reshape(-1)
    tiled = oracle.q4_k_row_tiled(raw, N, K)
    assert tiled.size == raw.size
    rows = raw.reshape(N, 74, 144)
    for g, s in [(0, 0), (0, 73), (100, 5), (255, 73)]:
        piece = tiled[(74 * g + s) * 2016:(74 * g + s + 1) * 2016].reshape(14, 144)
        assert np.array_equal(piece, rows[14 * g:14 * g + 14, s])


def test_refusals():
    raw = synth.random_blocks(oracle.Q4_K, 4, 4096, np.random.default_rng(2)).reshape(-1)
    with pytest.raises(ValueError):
        oracle.q4_k_row_tiled(raw, 4, 4096)          # 16 super-blocks: not a long row
    # 301 rows: two-row groups, the last one a real row and a filler row
    raw = synth.random_blocks(oracle.Q4_K, 301, 17 * 256, np.random.default_rng(3)).reshape(-1)
    tiled = oracle.q4_k_row_tiled(raw, 301, 17 * 256)
    assert tiled.size == 302 * 17 * 144
    with pytest.raises(ValueError):
        oracle.unpack_q4_k_row_tiled(tiled[:-1], 301, 17 * 256)
    bad = tiled.copy()
    bad[-1] = 1                                       # the filler row's last super-block
    with pytest.raises(ValueError):
        oracle.unpack_q4_k_row_tiled(bad, 301, 17 * 256)
