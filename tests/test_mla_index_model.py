"""Host-side model of the MLA-absorbed decode kernels' tile addressing for head counts that are
multiples of 64 (pairs of waves sharing 32 heads) and 128 (the wide kernel: 64 heads per pair of
waves, all heads of a row in one work-group); no GPU.

The formulas below restate, for every lane of the four waves, the index arithmetic of the pair
kernel in decode_mla.hip: the 16-byte chunk swizzle of the 576-dim cache rows, the direct-to-LDS
tile loads (slot -> tile row and chunk, clamp of the partial last tile), the LDS offsets of the
K operand reads (32x32x16 MFMA, k-step kk of reduction half r) and of the transposing V operand
reads (k-step ks, output block db of half r), and the partial-score exchange buffer. The checks
prove that every load stays inside its sequence's rows and its LDS stage, that the loads fill a
stage exactly once, that every operand read returns the logical element the product expects,
that the K-slot order of the P operand (taken from the score accumulator layout) matches the V
operand's, and that the reads are free of LDS bank conflicts under the gfx950 bank model the
kernels are tuned with (128-bit reads in four passes of 16 lanes selected by lane bit 5 and the
parity of lane bits 2-4; 64-bit reads in two passes of 32 lanes; a conflict is two lanes of a
pass on different 16-byte / 8-byte units of the same bank group). For the wide kernel: its
work-group id map (every (sequence, chunk, head group) once, all of a sequence on one XCD), the
scalar-base load offsets with the clamp of the chunk's last tile, the K reads over all 576 dims,
the staging of its query rows through the ring, and the LDS staging of its output (round trip and
bank conflicts).
"""
import numpy as np
import pytest

DQ, DV, TT = 576, 512, 32
TILE = TT * DQ            # elements per tile
NSLOT = TILE * 2 // 1024  # 36 load instructions of 1 KiB
WAVES, SPW = 4, 9


def key(row):
    return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1)


def tile_loads():
    """(wave, lane, slot, LDS element offset, tile row, logical chunk fetched)."""
    out = []
    for w in range(WAVES):
        for u in range(SPW):
            sl = w * SPW + u
            for lane in range(64):
                ob = sl * 1024 + 16 * lane
                row, pc = ob // (DQ * 2), (ob % (DQ * 2)) // 16
                out.append((w, lane, sl, sl * 512 + lane * 8, row, pc ^ key(row), pc))
    return out


def logical_tile():
    """tile[row][dim] = a unique id per element, and the LDS image the loads produce."""
    tile = np.arange(TILE, dtype=np.int64).reshape(TT, DQ)
    lds = np.full(TILE, -1, np.int64)
    for _, _, _, off, row, lc, _ in tile_loads():
        lds[off:off + 8] = tile[row, lc * 8:lc * 8 + 8]
    return tile, lds


def k_offsets(lane, r):
    col, hf = lane & 31, lane >> 5
    return [col * DQ + (((36 * r + hf + 2 * u) ^ key(col)) << 3) for u in range(4)]


def k_read(lane, r, kk):
    return k_offsets(lane, r)[kk & 3] + 64 * (kk >> 2)


def v_reads(lane, r, ks, db):
    """Element offsets of the two transposing reads (t = 0, 1) a lane issues for (ks, db)."""
    hf, tj, tc, dq = lane >> 5, (lane & 15) >> 2, lane & 3, (lane >> 4) & 1
    x = 2 * dq + (tc >> 1)
    vb = [[(4 * hf + tj) * DQ + 8 * (32 * r + 4 * (par ^ (tj >> 1)) + (x ^ (2 * hf) ^ t)) + (tc & 1) * 4
           for t in range(2)] for par in range(2)]
    base = 16 * ks * DQ + 32 * (db & ~1)
    return base + vb[db & 1][0], base + 8 * DQ + vb[db & 1][1]


def tr_read(lds, offs):
    """ds_read_b64_tr_b16 over a wave: in each 16-lane group, lanes 4j..4j+3 address 4 elements of
    row j; afterwards lane i of the group holds element i of rows 0..3."""
    out = np.empty((64, 4), np.int64)
    for g in range(4):
        rows = [[lds[offs[g * 16 + 4 * j + c] + e] for c in range(4) for e in range(4)] for j in range(4)]
        for i in range(16):
            out[g * 16 + i] = [rows[j][i] for j in range(4)]
    return out


def test_tile_loads_fill_each_stage_once():
    loads = tile_loads()
    assert sorted(off for *_, off, _, _, _ in [(l[0], l[1], l[2], l[3], l[4], l[5], l[6]) for l in loads]) == \
        list(range(0, TILE, 8))
    for row in range(TT):
        assert sorted(lc for *_, r, lc, _ in loads if r == row) == list(range(DQ // 8))
    for _, _, _, off, row, _, pc in loads:
        assert off == row * DQ + pc * 8
    # each wave issues exactly SPW loads per tile
    assert {w: sum(1 for l in loads if l[0] == w) // 64 for w in range(WAVES)} == {w: SPW for w in range(WAVES)}


@pytest.mark.parametrize("t0,t1", [(0, 1), (0, 45), (32, 64), (1024, 2048), (96, 130), (0, 4096)])
def test_tile_rows_stay_in_the_chunk(t0, t1):
    n_tiles = (t1 - t0 + TT - 1) // TT
    for j in range(n_tiles + 2):  # the ring re-reads the last tile past the end
        jj = min(j, n_tiles - 1)
        for _, _, _, _, row, lc, _ in tile_loads():
            t = min(t0 + jj * TT + row, t1 - 1)
            assert t0 <= t < t1
            assert 0 <= lc * 8 and lc * 8 + 8 <= DQ


def test_k_operand_reads_logical_elements():
    tile, lds = logical_tile()
    for r in range(2):
        for kk in range(18):
            for lane in range(64):
                off = k_read(lane, r, kk)
                assert 0 <= off and off + 8 <= TILE
                row, d0 = lane & 31, 288 * r + 16 * kk + 8 * (lane >> 5)
                assert list(lds[off:off + 8]) == list(tile[row, d0:d0 + 8]), (r, kk, lane)


def test_v_operand_reads_logical_elements():
    """A operand of O^T += V^T P^T: lane l holds dim 256r + 32db + (l & 31) at the tokens of k-slots
    8(l>>5) + e, which must be the tokens the score accumulator puts in the P operand's slots."""
    tile, lds = logical_tile()
    for r in range(2):
        for ks in range(2):
            for db in range(8):
                offs = [v_reads(lane, r, ks, db) for lane in range(64)]
                for t in range(2):
                    for lane in range(64):
                        assert 0 <= offs[lane][t] and offs[lane][t] + 4 <= TILE
                lo = tr_read(lds, [o[0] for o in offs])
                hi = tr_read(lds, [o[1] for o in offs])
                for lane in range(64):
                    hf = lane >> 5
                    dim = 256 * r + 32 * db + (lane & 31)
                    got = list(lo[lane]) + list(hi[lane])
                    # P operand slot e of k-step ks = score register v = 8ks + e of the accumulator,
                    # whose token is 8(v>>2) + 4hf + (v&3)
                    toks = [8 * ((8 * ks + e) >> 2) + 4 * hf + ((8 * ks + e) & 3) for e in range(8)]
                    assert got == [tile[tk, dim] for tk in toks], (r, ks, db, lane)


def _pass_conflicts(addrs_bytes, unit, groups):
    """Number of extra cycles: max over bank groups of distinct units addressed, minus one."""
    by_group = {}
    for a in addrs_bytes:
        u = a // unit
        by_group.setdefault(u % groups, set()).add(u)
    return max(len(v) for v in by_group.values()) - 1


def test_operand_reads_are_bank_conflict_free():
    for r in range(2):
        for kk in range(18):
            offs = [2 * k_read(lane, r, kk) for lane in range(64)]
            for b5 in range(2):
                for par in range(2):
                    lanes = [l for l in range(64) if (l >> 5) == b5 and bin((l >> 2) & 7).count("1") % 2 == par]
                    assert len(lanes) == 16
                    assert _pass_conflicts([offs[l] for l in lanes], 16, 16) == 0, (r, kk, b5, par)
        for ks in range(2):
            for db in range(8):
                offs = [v_reads(lane, r, ks, db) for lane in range(64)]
                for t in range(2):
                    for half in range(2):
                        addrs = [2 * offs[l][t] for l in range(32 * half, 32 * half + 32)]
                        assert _pass_conflicts(addrs, 8, 32) == 0, (r, ks, db, t, half)


def test_exchange_buffer_layout():
    """Partner waves (w, w^1) hold the same heads and tokens in the same lanes: the 16 scores of a
    lane go to xch[w][g][lane][0..3], g = v >> 2, and are read back from xch[w ^ 1] at the same
    place; the four 1 KiB rows of a wave are written by 128-bit stores of consecutive lanes."""
    seen = set()
    for w in range(WAVES):
        for g in range(4):
            for lane in range(64):
                base = ((w * 4 + g) * 64 + lane) * 4
                for i in range(4):
                    assert base + i not in seen
                    seen.add(base + i)
    assert seen == set(range(WAVES * 4 * 64 * 4))


# ---- the 128-heads-per-work-group kernel (head counts that are multiples of 128) ----

def wide_id_map(B, nsplit, n_hg):
    """Work-group id -> (sequence, chunk, head group) or None, as the wide kernel computes it."""
    n_wg = 8 * ((B + 7) // 8) * nsplit * n_hg
    out = []
    for i in range(n_wg):
        kx = i // 8
        hg, k2 = kx % n_hg, kx // n_hg
        b, s = i % 8 + 8 * (k2 // nsplit), k2 % nsplit
        out.append(None if b >= B else (b, s, hg))
    return out


@pytest.mark.parametrize("B,nsplit,n_hg", [(1, 1, 1), (3, 8, 1), (8, 8, 1), (9, 3, 2), (32, 8, 1), (33, 5, 2),
                                           (256, 1, 1)])
def test_wide_grid_covers_every_unit_once_on_one_xcd(B, nsplit, n_hg):
    m = wide_id_map(B, nsplit, n_hg)
    units = [u for u in m if u is not None]
    assert sorted(units) == [(b, s, g) for b in range(B) for s in range(nsplit) for g in range(n_hg)]
    # every chunk and head group of a sequence runs on the XCD of id % 8 == b % 8
    for i, u in enumerate(m):
        if u is not None:
            assert i % 8 == u[0] % 8


def wide_slot_offsets(w, lane, ldk):
    """Per slot u: (tile row, logical chunk, byte offset of the full-tile load) of wave w's lane."""
    out = []
    for u in range(SPW):
        ob = (w * SPW + u) * 1024 + 16 * lane
        row, pc = ob // (DQ * 2), (ob % (DQ * 2)) // 16
        lc = pc ^ key(row)
        out.append((row, lc, 2 * (row * ldk + lc * 8)))
    return out


@pytest.mark.parametrize("ldk", [576, 640, 4096])
@pytest.mark.parametrize("lim", [31, 30, 17, 0])
def test_wide_scalar_base_offsets_clamp_rows(ldk, lim):
    """Full tiles: base + loff; the chunk's last tile (last valid row lim < 31): rows past lim read
    row lim, i.e. loff - 2(row - lim) ldk. Every byte offset is the pointer form's, inside the
    tile's valid rows, and fits the 32-bit offset operand."""
    for w in range(WAVES):
        for lane in range(64):
            for row, lc, off in wide_slot_offsets(w, lane, ldk):
                assert 0 <= lc < DQ // 8
                got = off if row <= lim else off - 2 * (row - lim) * ldk
                want = 2 * (min(row, lim) * ldk + lc * 8)
                assert got == want
                assert 0 <= got and got + 16 <= 2 * (lim * ldk + DQ) and got < 2 ** 31


def test_wide_k_operand_reads_all_576_dims():
    """K operand of k-step kk (0..35), the whole row of the own heads: row col, dims 16kk + 8hf."""
    tile, lds = logical_tile()
    for kk in range(36):
        for lane in range(64):
            col, hf = lane & 31, lane >> 5
            off = col * DQ + (((2 * (kk & 3) + hf) ^ key(col)) << 3) + 64 * (kk >> 2)
            assert 0 <= off and off + 8 <= TILE
            assert list(lds[off:off + 8]) == list(tile[col, 16 * kk + 8 * hf:16 * kk + 8 * hf + 8]), (kk, lane)


def test_wide_output_staging_round_trip_and_banks():
    """The output of a wave (64 rows x 256 dims, bf16) is written to LDS by 64-bit stores (lane
    (col, hf) of group g: row 32g + col, chunk 4db + e, half hf) at chunk c ^ (row & 31), half
    hf ^ bit 4 of the row, then read back by 128-bit loads (lane: row 2i + hf, chunk col) and the
    halves swapped back: every element lands once and comes back where the stores expect it, and
    both access patterns are free of bank conflicts."""
    lds = {}
    for g in range(2):
        for db in range(8):
            for e in range(4):
                addrs = []
                for lane in range(64):
                    col, hf = lane & 31, lane >> 5
                    hl, c = 32 * g + col, 4 * db + e
                    a = hl * 256 + ((c ^ (hl & 31)) << 3) + ((hf ^ ((hl >> 4) & 1)) << 2)
                    for i in range(4):
                        assert a + i not in lds
                        lds[a + i] = (hl, 8 * c + 4 * hf + i)  # (row, dim) of the value
                    addrs.append(2 * a)
                for half in range(2):  # 64-bit accesses: two passes of 32 lanes
                    assert _pass_conflicts(addrs[32 * half:32 * half + 32], 8, 32) == 0
    assert sorted(lds) == list(range(64 * 256))
    for i in range(32):
        addrs = []
        for lane in range(64):
            col, hf = lane & 31, lane >> 5
            hl = 2 * i + hf
            a = hl * 256 + ((col ^ (hl & 31)) << 3)
            v = [lds[a + k] for k in range(8)]
            if (hl >> 4) & 1:
                v = v[4:] + v[:4]
            assert v == [(hl, 8 * col + k) for k in range(8)]
            addrs.append(2 * a)
        for b5 in range(2):
            for par in range(2):
                lanes = [l for l in range(64) if (l >> 5) == b5 and bin((l >> 2) & 7).count("1") % 2 == par]
                assert _pass_conflicts([addrs[l] for l in lanes], 16, 16) == 0


def test_wide_query_staging_through_the_ring():
    """The wide kernel's query rows: wave w's 32 rows (36 KiB, contiguous) are loaded like a tile
    (slot u, lane i: bytes 1024u + 16i = row * 1152 + 16pc, logical chunk pc ^ key(row)) into stage
    u & 3 at 1-KiB column 9w + (u >> 2); k-step kk is read back at the tile position of (row col,
    chunk 2kk + hf). Every load reads inside the wave's rows, lands once inside the wave's own
    columns (the ones its tile loads refill later, so no other wave touches them), every read
    returns q[col][16kk + 8hf .. +7], and the reads are free of bank conflicts (the remap moves
    whole 1-KiB slots, so the bank pattern is the K reads')."""
    STAGE = TILE  # elements per ring stage
    for w in range(WAVES):
        lds = {}
        for u in range(NSLOT):
            for lane in range(64):
                ob = u * 1024 + 16 * lane
                row, pc = ob // (DQ * 2), (ob % (DQ * 2)) // 16
                src = row * DQ + ((pc ^ key(row)) << 3)  # element offset within the wave's rows
                assert 0 <= src and src + 8 <= 32 * DQ
                dst = (u & 3) * STAGE + (9 * w + (u >> 2)) * 512 + lane * 8
                assert (dst % STAGE) // (9 * 512) == w  # this wave's column of the stage
                for k in range(8):
                    assert dst + k not in lds
                    lds[dst + k] = src + k
        # the same columns are the ones wave w's tile loads fill: slots 9w .. 9w + 8 of every stage
        cols = {(d % STAGE) // 512 for d in lds}
        assert cols == set(range(9 * w, 9 * w + 9))
        for kk in range(36):
            addrs = []
            for lane in range(64):
                col, hf = lane & 31, lane >> 5
                bq = col * (DQ * 2) + 16 * (8 * (kk >> 2) + ((2 * (kk & 3) + hf) ^ key(col)))
                u = bq >> 10
                a = (u & 3) * STAGE + (9 * w + (u >> 2)) * 512 + ((bq & 1023) >> 1)
                assert [lds[a + k] for k in range(8)] == [col * DQ + 16 * kk + 8 * hf + k for k in range(8)]
                addrs.append(2 * a)
            for b5 in range(2):
                for par in range(2):
                    lanes = [l for l in range(64) if (l >> 5) == b5 and bin((l >> 2) & 7).count("1") % 2 == par]
                    assert _pass_conflicts([addrs[l] for l in lanes], 16, 16) == 0


def test_wide_rope_pairs_and_residual_operands():
    """In-kernel q^R RoPE in the wide kernel: lane (col, hf) holds dims 16kk + 8hf .. +7 in query
    register kk, so the rotation partners 512 + i and 544 + i (i = 16u + 8hf + j) sit in the same
    lane, in registers 32 + u and 34 + u (u = 0, 1), with i0 = 16u + 8hf as the rotation is called.
    After the 36-step chain with four K operands in flight (slot kk % 4 refilled with k-step kk + 4
    while kk + 4 < 36), slot (32 + u) % 4 still holds k-step 32 + u: the residual products pair the
    residual of register 32 + u with the K dims it was rotated for."""
    DV_ = 512
    for hf in range(2):
        for u in range(2):
            i0 = 16 * u + 8 * hf
            for j in range(8):
                a = 16 * (32 + u) + 8 * hf + j
                b = 16 * (34 + u) + 8 * hf + j
                assert a == DV_ + i0 + j and b == DV_ + 32 + i0 + j
    KR, KS = 4, 36
    slot = [kk for kk in range(KR)]
    for kk in range(KS):
        assert slot[kk % KR] == kk  # the product of k-step kk reads its own K operand
        if kk + KR < KS:
            slot[kk % KR] = kk + KR
    for u in range(4):
        assert slot[(KS - 4 + u) % KR] == KS - 4 + u
