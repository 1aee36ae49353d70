"""CPU pins of the LDS sizes the kernels are built and launched with.

mq_debug_lds_bytes reports, from the host, the sizes the library computes from its
own formulas and structs; each is compared here with the size written out from the
layout the kernel's comments describe, and with the 160 KiB of LDS a gfx950 CU has
("minfer CUDA Backend Design", 2.4: one shared-memory formula per kernel, gated by
tests)."""

import pytest

from block_quantized_matmul_mq_amd import mq

LIMIT = 160 * 1024
FIXED, TILE_UNITS, I8_BM128, I8_BM32, F6, KW = 0, 1, 2, 3, 5, 6
TYPES = [mq.Q4_0, mq.Q4_1, mq.Q5_0, mq.Q5_1, mq.Q8_0, mq.Q4_K, mq.Q5_K, mq.Q6_K]
KQUANT = {mq.Q4_K, mq.Q5_K, mq.Q6_K}
MIN_TERM = {mq.Q4_1, mq.Q5_1, mq.Q4_K, mq.Q5_K}   # a per-block min is subtracted


def lds(what, qtype, K=0):
    return mq.load().mq_debug_lds_bytes(what, qtype, K)


def gemv_fixed_expected(qtype, K):
    # three digit planes, each (units + 1) rows of 16-byte chunks per 16 values of a unit;
    # then int32 block exponents and f32 sums: per 32-block, or per (unit, 16-run) for Q6_K
    vals = 64 if qtype in KQUANT else 32
    U = K // vals
    planes = 3 * (vals // 16) * (U + 1) * 16
    if qtype == mq.Q6_K:
        return planes + 4 * U * 4 + 4 * U * 4
    return planes + (K // 32) * 4 + (0 if qtype == mq.Q8_0 else (K // 32) * 4)


@pytest.mark.parametrize("qtype", TYPES, ids=[str(t) for t in TYPES])
def test_vector_gemv_lds(qtype):
    block = 256 if qtype in KQUANT else 32
    for K in sorted({block, 2 * block, 896, 3584, 4864, 5120, 13824, 18944, 27648, 32768}):
        if K % block:
            continue
        fixed = lds(FIXED, qtype, K)
        assert fixed == gemv_fixed_expected(qtype, K), (qtype, K)
        U = K // (64 if qtype in KQUANT else 32)
        units = lds(TILE_UNITS, qtype, K)
        if fixed + 4 * U <= LIMIT:
            # at least one row of partials, everything inside the CU's LDS, and the
            # largest such tile (capped at 65536 units)
            assert units >= U and fixed + 4 * units <= LIMIT, (qtype, K, units)
            assert units == 65536 or fixed + 4 * (units + 1) > LIMIT
        else:
            assert units == 0
    # every K the calls accept fits one row at the largest K
    assert lds(TILE_UNITS, qtype, 32768) > 0
    assert lds(FIXED, qtype, 100) == 0 and lds(99, qtype, 256) == 0


@pytest.mark.parametrize("qtype", TYPES, ids=[str(t) for t in TYPES])
def test_int8_mmq_lds(qtype):
    # double-buffered: codes A [bm][128] and B [128][128] (int8), activation scales
    # [4 blocks][bm] f32, min-term operands [4 or 1][bm] u32, weight scales [4 blocks, or 8
    # 16-groups for Q6_K][128] f32, weight min operands [4 or 1][128] u32
    for what, bm in [(I8_BM128, 128), (I8_BM32, 32)]:
        nmin = 4 if qtype in MIN_TERM else 1
        groups = 8 if qtype == mq.Q6_K else 4
        want = 2 * (bm * 128 + 128 * 128 + 4 * bm * 4 + nmin * bm * 4 + groups * 128 * 4 + nmin * 128 * 4)
        got = lds(what, qtype)
        assert got == want, (qtype, bm, got, want)
        assert 2 * got <= LIMIT, "two workgroups per CU (512 resident) is what the work split assumes"


def test_fp6_mmq_lds():
    # ring of 3 step slots, each one step of both planes for a 128 x 128 tile: activation
    # rows 128 x (64 B of digit records + 32 B of their tails + 8 B dx pairs x 2 blocks + 8 B
    # min pairs x 2 blocks), weight rows 128 x (32 + 16 + 16 + 16 B); plus a 1 KB sink for
    # the loads that carry nothing
    slot = 128 * (64 + 32 + 16 + 16) + 128 * (32 + 16 + 16 + 16)
    assert slot == 26 * 1024
    assert lds(F6, mq.Q4_K) == 3 * slot + 1024
    assert 2 * lds(F6, mq.Q4_K) <= LIMIT, "two workgroups per CU (512 resident) is what the work split assumes"
    assert lds(F6, mq.Q8_0) == 0


def test_k_over_waves_mmq_lds():
    # the four waves' f32 partial tiles of 32 x 32 (16 accumulator elements x 64 lanes
    # each) meet in LDS for the final sum; nothing else is staged there
    assert lds(KW, mq.Q4_K) == 4 * 16 * 64 * 4
    assert 2 * lds(KW, mq.Q4_K) <= LIMIT, "two workgroups per CU"
    assert lds(KW, mq.Q8_0) == 0
