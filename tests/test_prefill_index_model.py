"""Host-side model of the bf16 prefill kernel's tile addressing (no GPU).

The formulas below restate, for every lane, the index arithmetic of prefill_bf16.hip: the 16-byte
chunk swizzle, the direct-to-LDS tile loads (slot -> tile row and chunk), the clamp of the partial
last tile, and the LDS offsets of the K operand reads and of the transposing V operand reads. The
checks prove, for each head-dim pair the library builds - (64, 64), (128, 128) and MLA's (192, 128) -
that every load stays inside its tensor slice and its LDS stage, that the loads fill each stage
exactly once, and that every operand read lands on the logical element the MFMA step expects.
"""
import numpy as np
import pytest

KBC = 32  # keys per tile


def swz(ch, c, row):
    if ch == 24:
        return c ^ (((row >> 1) & 1) | (((row >> 3) & 1) << 1) | (((row >> 4) & 1) << 2))
    key = ((row & 3) << 1) | ((row >> 2) & 1) | ((row & 8) if ch == 16 else 0)
    return c ^ key


def tile_loads(d):
    """(LDS element offset, tile row, logical chunk) of every lane's 16 bytes, over the 4 waves."""
    lp = KBC * (d // 8) // 64 // 4
    out = []
    for w in range(4):
        for r in range(lp):
            sl = w * lp + r
            for lane in range(64):
                b = sl * 1024 + 16 * lane
                row, pc = b // (d * 2), (b % (d * 2)) // 16
                out.append((sl * 512 + lane * 8, row, swz(d // 8, pc, row), pc))
    return out


DIMS = [(64, 64), (128, 128), (192, 128)]


@pytest.mark.parametrize("dqk,dv", DIMS)
def test_tile_loads_fill_each_stage_once(dqk, dv):
    for d in (dqk, dv):
        loads = tile_loads(d)
        lds = sorted(o for o, *_ in loads)
        assert lds == list(range(0, KBC * d, 8))  # 8 elements per lane, no gap, no overlap
        # physical chunk pc of row holds logical chunk swz(pc): a bijection per row
        for row in range(KBC):
            logical = sorted(lc for _, r, lc, _ in loads if r == row)
            assert logical == list(range(d // 8)), (d, row)
        for off, row, lc, pc in loads:
            assert off == row * d + pc * 8  # the LDS stage stores rows as in memory, chunks permuted


@pytest.mark.parametrize("dqk,dv", DIMS)
@pytest.mark.parametrize("sk", [1, 31, 32, 33, 200, 4096])
def test_partial_tile_reads_stay_in_the_sequence(dqk, dv, sk):
    n_tiles = (sk + KBC - 1) // KBC
    for d in (dqk, dv):
        for jt in range(n_tiles):
            full = jt * KBC + KBC <= sk
            for _, row, lc, _ in tile_loads(d):
                key = jt * KBC + row if full else min(jt * KBC + row, sk - 1)
                assert 0 <= key < sk
                assert 0 <= lc * 8 and lc * 8 + 8 <= d


@pytest.mark.parametrize("dqk,dv", DIMS)
def test_k_operand_reads(dqk, dv):
    ch = dqk // 8
    for lane in range(64):
        col, hh = lane & 31, lane >> 5
        kb_lane = col * dqk + swz(ch, hh, col) * 8
        for kk in range(dqk // 16):
            koff = col * dqk + swz(ch, 2 * kk + hh, col) * 8
            if dqk <= 128:
                assert koff == kb_lane ^ (16 * kk)  # the kernel's register-free form
            row, pc = koff // dqk, (koff % dqk) // 8
            assert row == col and swz(ch, pc, row) == 2 * kk + hh
            assert 0 <= koff and koff + 8 <= KBC * dqk


@pytest.mark.parametrize("dv", [64, 128])
def test_v_transposing_reads(dv):
    ch = dv // 8
    for lane in range(64):
        hh, tr_dq, tr_j, tr_c = lane >> 5, (lane >> 4) & 1, (lane & 15) >> 2, lane & 3
        voff_par = []
        for par in range(2):
            row = hh * 4 + tr_j
            voff_par.append(row * dv + swz(ch, par * 4 + tr_dq * 2 + (tr_c >> 1), row) * 8 + (tr_c & 1) * 4)
        for s in range(2):
            for t in range(2):
                for db in range(dv // 32):
                    dbase = (db & ~1) * 32
                    tshift = (-64 if (db >> 1) & 1 else 64) if ch == 16 else 0
                    a = 16 * s * dv + voff_par[db & 1] + dbase + t * (8 * dv + tshift)
                    row, e = a // dv, a % dv
                    logical = swz(ch, e // 8, row) * 8 + e % 8
                    assert row == 16 * s + 8 * t + hh * 4 + tr_j, (dv, lane, s, t, db)
                    assert logical == db * 32 + tr_dq * 16 + 4 * tr_c, (dv, lane, s, t, db)
                    assert 0 <= a and a + 4 <= KBC * dv


def test_swizzle_is_a_permutation_per_row():
    for ch in (8, 16, 24):
        for row in range(KBC):
            assert sorted(swz(ch, c, row) for c in range(ch)) == list(range(ch))
