"""Host model of the GQA decode kernel's work-item order (csrc/decode.hip, decode_item).

The split kernel's work-groups are dispatched in the order: every sequence's full chunks
(sequence-major), then the short last chunks of the sequences whose context is not a multiple of the
chunk, also sequence-major. The model below replays the kernel's wave-level steps (a 64-lane
inclusive scan per block of sequences, ballots, the j-th set bit) lane by lane on the CPU and checks
that the items 0 .. B*nsplit-1 cover every non-empty (sequence, chunk) exactly once, in that order,
and that the rest report "past the last item". No GPU is needed.
"""
import numpy as np
import pytest

LANES = 64


def clamp_ctx(ctx_lens, max_ctx, b0):
    lane = np.arange(LANES)
    b = b0 + lane
    ctx = np.zeros(LANES, dtype=np.int64)
    ok = b < len(ctx_lens)
    ctx[ok] = np.clip(np.asarray(ctx_lens)[b[ok]], 0, max_ctx)
    return ctx


def decode_item(ctx_lens, max_ctx, chunk, item):
    """Lane-level replay of the kernel's item -> (b, s) mapping; None past the last item."""
    B = len(ctx_lens)
    lane = np.arange(LANES)
    before = 0
    for b0 in range(0, B, LANES):
        ctx = clamp_ctx(ctx_lens, max_ctx, b0)
        f = ctx // chunk
        incl = f.copy()
        d = 1
        while d < LANES:  # shfl_up scan: lanes below d keep their value
            y = np.concatenate([incl[:d], incl[:-d]])
            incl = np.where(lane >= d, incl + y, incl)
            d <<= 1
        total = int(incl[63])
        if item < before + total:
            mask = (before + incl) > item
            l = int(np.argmax(mask))  # lowest set lane of the ballot
            return b0 + l, int(item - before - (incl[l] - f[l]))
        before += total
    j = item - before
    for b0 in range(0, B, LANES):
        ctx = clamp_ctx(ctx_lens, max_ctx, b0)
        part = (ctx % chunk) != 0
        cnt = int(part.sum())
        if j < cnt:
            below = np.array([part[:i].sum() for i in range(LANES)])
            hit = part & (below == j)
            l = int(np.argmax(hit))
            return b0 + l, int(ctx[l] // chunk)
        j -= cnt
    return None


def expected_order(ctx_lens, max_ctx, chunk):
    ctx = np.clip(np.asarray(ctx_lens), 0, max_ctx)
    full = [(b, s) for b in range(len(ctx)) for s in range(int(ctx[b]) // chunk)]
    short = [(b, int(ctx[b]) // chunk) for b in range(len(ctx)) if ctx[b] % chunk]
    return full + short


CASES = [
    # (B, chunk, max_ctx, context recipe)
    (64, 1024, 8192, "uniform"),     # the Llama-3-8B decode shape
    (5, 1024, 3000, "uniform"),
    (130, 256, 2048, "uniform"),     # three blocks of 64 sequences
    (70, 512, 4096, "multiples"),    # no short chunks at all
    (9, 64, 700, "with_empty"),      # empty and negative contexts, lengths past max_ctx
    (1, 1024, 1, "uniform"),
]


@pytest.mark.parametrize("B,chunk,max_ctx,recipe", CASES)
def test_items_cover_every_chunk_once_longest_first(B, chunk, max_ctx, recipe):
    rng = np.random.default_rng(B * 7 + chunk)
    if recipe == "uniform":
        ctx = rng.integers(1, max_ctx + 1, B)
    elif recipe == "multiples":
        ctx = rng.integers(1, max_ctx // chunk + 1, B) * chunk
    else:
        ctx = rng.integers(-3, max_ctx + 200, B)
        ctx[::3] = 0
    nsplit = -(-max_ctx // chunk)
    got = [decode_item(ctx, max_ctx, chunk, i) for i in range(B * nsplit)]
    want = expected_order(ctx, max_ctx, chunk)
    assert got[:len(want)] == want
    assert all(g is None for g in got[len(want):])
    # every item maps inside the grid's (sequence, split) range and before the context end
    ctxc = np.clip(ctx, 0, max_ctx)
    for b, s in want:
        assert 0 <= b < B and 0 <= s < nsplit and s * chunk < ctxc[b]


@pytest.mark.parametrize("nhg", [8, 16, 1, 2, 4, 3])
def test_head_groups_rotate_over_xcds_and_cover_each_item(nhg):
    """The GQA split kernel's head group of work-group id: (id + b) % nhg, where b is the sequence of
    item id // nhg. Every item's nhg work-groups take every head group once (nothing skipped,
    nothing twice), and with 8 KV heads the XCD of an id (id % 8) reads different KV heads for
    different sequences instead of one fixed 256-byte slice of every cache row."""
    ctx = np.array([5000, 1024, 8192, 3000, 17, 4096, 2048, 6000, 7000], np.int32)
    max_ctx, chunk = 8192, 1024
    nsplit = max_ctx // chunk
    seen_by_xcd = {x: set() for x in range(8)}
    for item in range(len(ctx) * nsplit):
        it = decode_item(ctx, max_ctx, chunk, item)
        if it is None:
            continue
        b, s = it
        hg = [(item * nhg + t + b) % nhg for t in range(nhg)]
        assert sorted(hg) == list(range(nhg))
        for t in range(nhg):
            seen_by_xcd[(item * nhg + t) % 8].add(hg[t])
    if nhg == 8:
        assert all(len(v) == 8 for v in seen_by_xcd.values())
