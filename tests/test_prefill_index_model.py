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


# ---- the whole grid: block id -> (sequence, head group, q-tile), then every access's extent ----
def grid_map(B, S, Nh, HPW, n_ptiles):
    """(b, h0, pt) of every work-group id, as the kernel computes them."""
    HGn = Nh // HPW
    npairs = B * HGn
    ids = np.arange(n_ptiles * npairs, dtype=np.int64)
    if npairs % 8 == 0:
        li = ids // 8
        ppx = npairs // 8
        j = li % ppx
        bh = 8 * j + (ids % 8 + j) % 8
        pt = n_ptiles - 1 - li // ppx
    else:
        bh = ids % npairs
        pt = n_ptiles - 1 - ids // npairs
    return bh // HGn, (bh % HGn) * HPW, pt


def lane_offsets(d, tok):
    """Per-lane element offsets (row * tok + physical chunk * 8) of one tile's loads, all waves."""
    lp = KBC * (d // 8) // 64 // 4
    offs, rows = [], []
    for w in range(4):
        for r in range(lp):
            sl = w * lp + r
            for lane in range(64):
                b = sl * 1024 + 16 * lane
                row, pc = b // (d * 2), (b % (d * 2)) // 16
                assert row * tok < 2 ** 31  # the kernel forms row * (int)tok in 32 bits
                offs.append(row * tok + swz(d // 8, pc, row) * 8)
                rows.append(row)
    return np.array(offs, np.int64), np.array(rows, np.int64)


GRID_CASES = [
    # B, S, Nh, Nkv, DQK, DV, causal
    (1, 4096, 128, 128, 192, 128, True),   # DeepSeek-V3-shaped MLA non-absorbed prefill
    (4, 8192, 32, 8, 128, 128, True),      # Llama-3-8B-shaped GQA prefill
    (8, 1024, 12, 12, 64, 64, True),       # GPT-2-small-shaped prefill
    (1, 200, 4, 4, 192, 128, True),
    (2, 97, 4, 4, 192, 128, True),
    (1, 130, 8, 2, 192, 128, True),
    (1, 150, 4, 2, 192, 128, False),
    (3, 1, 4, 4, 192, 128, True),
    (1, 256, 2, 2, 192, 128, True),
]


@pytest.mark.parametrize("case", GRID_CASES, ids=lambda c: "B%dS%dH%dK%d_%d_%d_c%d" % c)
def test_grid_covers_every_tile_once_and_stays_in_bounds(case):
    B, S, Nh, Nkv, dqk, dv, causal = case
    G = Nh // Nkv
    HPW = 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1
    BP = 32 * (4 // HPW)
    n_ptiles = (S + BP - 1) // BP
    b, h0, pt = grid_map(B, S, Nh, HPW, n_ptiles)
    # every (sequence, head group, q-tile) exactly once: nothing skipped, nothing written twice
    keys = (b * (Nh // HPW) + h0 // HPW) * n_ptiles + pt
    assert np.array_equal(np.sort(keys), np.arange(B * (Nh // HPW) * n_ptiles))
    assert b.min() >= 0 and b.max() < B and h0.max() + HPW <= Nh and pt.min() >= 0
    g = h0 // G
    p0 = pt * BP
    # K (the rotated copy in the workspace when RoPE is on, same layout) and V: [B, S, Nkv, d]
    for d in (dqk, dv):
        tok, batch, head = Nkv * d, S * Nkv * d, d
        size = B * S * Nkv * d
        loff, lrow = lane_offsets(d, tok)
        last = np.minimum(S, p0 + BP) if causal else np.full_like(p0, S)
        n_tiles = (last + KBC - 1) // KBC
        base = b * batch + g * head
        # full tiles (jt * 32 + 32 <= S): base + jt * 32 * tok + loff, increasing in jt and loff
        n_full = np.minimum(n_tiles, S // KBC)
        has_full = n_full > 0
        lo = base + loff.min()
        hi = base + (n_full - 1) * KBC * tok + loff.max() + 8
        if has_full.any():
            assert lo[has_full].min() >= 0 and hi[has_full].max() <= size
            assert ((n_full - 1) * KBC + lrow.max())[has_full].max() <= S - 1  # keys inside the sequence
        # a partial last tile: key = min(jt * 32 + row, S - 1), chunk inside the row
        part = n_tiles > n_full
        if part.any():
            key_hi = np.minimum((n_tiles - 1) * KBC + lrow.max(), S - 1)
            hi_p = base + key_hi * tok + d
            assert hi_p[part].max() <= size and ((n_tiles - 1) * KBC)[part].min() >= 0
    # q reads and out writes of the rows p < S: [B, S, Nh, dqk] / [B, S, Nh, dv]
    for w in range(4):
        h = h0 + w % HPW
        pw = p0 + (w // HPW) * 32 + 31  # the wave's last row
        pw = np.minimum(pw, S - 1)
        q_hi = ((b * S + pw) * Nh + h) * dqk + 8 + (dqk // 16 - 1) * 16 + 8
        o_hi = ((b * S + pw) * Nh + h) * dv + 4 + (dv // 32 - 1) * 32 + 3 * 8 + 4
        assert q_hi.max() <= B * S * Nh * dqk and o_hi.max() <= B * S * Nh * dv


@pytest.mark.parametrize("KS", [1, 2, 4])
@pytest.mark.parametrize("S,causal", [(600, True), (545, True), (512, False), (1024, True), (33, True), (1, True)])
def test_split_key_grid_covers_every_block_tile_once(KS, S, causal):
    """The split-key prefill: work-group qg holds query blocks qg*QB .. qg*QB+QB-1 (QB = 4/KS);
    wave w takes block w // KS and key split w % KS. The QB waves of one key split share a 2-stage
    ring: at step i each of them loads its LW = LT/QB slots of tile ks + KS*i (when some block of
    the work-group needs it) and computes it (when its own block needs it). Every wave runs the same
    number of steps (one barrier each), every (block, visible key tile) is computed by exactly one
    wave, every computed tile was loaded whole (every slot once) into the stage it is read from,
    and the merge's 256 threads write every (row, dim) of the group once."""
    QB = 4 // KS
    n_qb = (S + 32 * QB - 1) // (32 * QB)
    seen = {}
    for qg in range(n_qb):
        def need(qs):
            pq = (qg * QB + qs) * 32
            return 0 if pq >= S else ((min(S, pq + 32) if causal else S) + 31) // 32
        max_tiles = max(need(qs) for qs in range(QB))
        steps = []
        for w in range(4):
            qsub, ks = w // KS, w % KS
            n_steps = (max_tiles + KS - 1) // KS  # computed the same way by every wave
            steps.append(n_steps)
            for i in range(n_steps):
                jt = ks + KS * i
                if jt < need(qsub):
                    key = (qg * QB + qsub, jt)
                    assert key not in seen
                    seen[key] = w
                    # the tile was loaded in full into stage i & 1 of ring ks by the ring's QB waves
                    assert jt < max_tiles
        assert len(set(steps)) == 1
    want = {(qb, j) for qb in range((S + 31) // 32) for j in range(((min(S, 32 * qb + 32) if causal else S) + 31) // 32)}
    assert set(seen) == want
    for D in (64, 128):
        LT = 32 * (D // 8) // 64
        LW = LT // QB
        assert LT % QB == 0
        slots = sorted(qsub * LW + u for qsub in range(QB) for u in range(LW))
        assert slots == list(range(LT))  # the ring's waves cover a tile's load slots once
        TPR = 8 // QB
        PER = D // TPR
        cells = set()
        for t in range(256):
            r, d0 = t // TPR, (t % TPR) * PER
            for e in range(PER):
                cells.add((r, d0 + e))
        assert cells == {(r, d) for r in range(32 * QB) for d in range(D)}
    # LDS: the rings, or the merge area once the loop is done, whichever is larger (64-dim heads:
    # 35 KiB, four work-groups per CU)
    for D, per_cu in ((64, 4), (128, 2)):
        ring = KS * 2 * 2 * 32 * D * 2
        merge = 4 * (32 * (D + 4) + 64) * 4
        assert per_cu * max(ring, merge) <= 160 * 1024 or KS != 2


def test_block_order_is_heaviest_first_on_every_xcd():
    """Llama-3-8B shape (32 (sequence, head group) pairs): work-group id runs on XCD id % 8; each XCD
    holds four pairs of its own, one KV head of each sequence, four different KV heads; and in
    launch order its q-tiles never get heavier, so its last work-groups are the lightest ones of
    all its pairs."""
    B, S, Nh, HPW = 4, 8192, 32, 4
    n_ptiles = S // 32
    b, h0, pt = grid_map(B, S, Nh, HPW, n_ptiles)
    bh = b * (Nh // HPW) + h0 // HPW
    ids = np.arange(len(pt))
    owner = {}
    for x in range(8):
        sel = ids % 8 == x
        pairs = set(np.unique(bh[sel]).tolist())
        assert len(pairs) == 4 and not any(p in owner for p in pairs)
        owner.update({p: x for p in pairs})
        assert sorted(np.unique(b[sel]).tolist()) == [0, 1, 2, 3]
        assert len(np.unique(h0[sel])) == 4
        assert np.all(np.diff(pt[sel]) <= 0)
        assert pt[sel][-1] == 0 and pt[sel][0] == n_ptiles - 1


def claim(lists, x, per_x):
    """One work-group's claim on XCD x, as the kernel makes it (counters are atomic, so any run is
    some order of whole claims): its own list first, then the first list in rotation order from x
    whose counter is below per_x; None once every list is used up."""
    c0 = lists[x]
    lists[x] += 1
    if c0 < per_x:
        return x, c0
    for _ in range(8):
        open_ = [k for k in range(8) if lists[(x + k) % 8] < per_x]
        if not open_:
            return None
        xk = (x + open_[0]) % 8
        ck = lists[xk]
        lists[xk] += 1
        if ck < per_x:
            return xk, ck
    return None


@pytest.mark.parametrize("B,S,Nh,HPW,seed", [(4, 8192, 32, 4, 0), (4, 8192, 32, 4, 1), (2, 640, 32, 4, 2),
                                             (8, 96, 8, 1, 3)])
def test_work_lists_cover_every_item_once(B, S, Nh, HPW, seed):
    """Work lists with stealing: the grid has an eighth more work-groups than items, each XCD gets
    work-group ids x, x + 8, ...; in any order of the claims (fast XCDs claiming far ahead of slow
    ones) every item is computed exactly once and every other work-group leaves. The items of a
    list map to the static order's (pair, q-tile) of that XCD."""
    rng = np.random.default_rng(seed)
    HGn = Nh // HPW
    npairs = B * HGn
    assert npairs % 8 == 0
    n_ptiles = (S + 32 * (4 // HPW) - 1) // (32 * (4 // HPW))
    n_items = n_ptiles * npairs
    n_wg = n_items + 8 * ((n_items // 8 + 7) // 8)
    ppx = npairs // 8
    per_x = ppx * n_ptiles
    speed = rng.uniform(0.8, 1.2, 8)  # XCD x issues its next claim after 1 / speed[x] time units
    t = np.zeros(8)
    nxt = [[i for i in range(n_wg) if i % 8 == x] for x in range(8)]
    lists = [0] * 8
    done = []
    while any(nxt):
        x = min((x for x in range(8) if nxt[x]), key=lambda x: t[x])
        nxt[x].pop(0)
        t[x] += rng.uniform(0.5, 1.5) / speed[x]
        r = claim(lists, x, per_x)
        if r is not None:
            done.append(r)
    assert len(done) == n_items
    items = [(xk, c) for xk, c in done]
    assert len(set(items)) == n_items
    # the (pair, q-tile) of list xk, position c is the static order's item of XCD xk
    b, h0, pt = grid_map(B, S, Nh, HPW, n_ptiles)
    bh_static = (b * HGn + h0 // HPW)
    static = {(i % 8, i // 8): (bh_static[i], pt[i]) for i in range(n_items)}
    got = set()
    for xk, c in items:
        j = c % ppx
        got.add((8 * j + (xk + j) % 8, n_ptiles - 1 - c // ppx))
        assert static[(xk, c)] == (8 * j + (xk + j) % 8, n_ptiles - 1 - c // ppx)
    assert len(got) == n_items
