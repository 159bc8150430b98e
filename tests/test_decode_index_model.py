"""Host model of the GQA decode kernel's chunks and work-item order (csrc/decode.hip, chunk_plan and
decode_item).

A context of ctx tokens is n = ceil(ctx / chunk) chunks of ceil(ctx / n) tokens (the last one shorter
by less than n), so every chunk of a context longer than one chunk holds chunk/2 .. chunk tokens. The
split kernel's work-groups are dispatched sequence-major, the chunks of a sequence together. The model
below replays the kernel's wave-level steps (a 64-lane inclusive scan per block of sequences, ballots)
lane by lane on the CPU and checks that the items 0 .. B*nsplit-1 cover every (sequence, chunk)
exactly once, in that order, that the chunks tile each context, and that the rest report "past the
last item". No GPU is needed.
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


def chunk_plan(ctx, chunk):
    """(count, length) of a context's chunks, as the kernel computes them."""
    n = -(-ctx // chunk)
    length = -(-ctx // n) if n > 0 else 0
    return n, length


def decode_item(ctx_lens, max_ctx, chunk, item):
    """Lane-level replay of the kernel's item -> (b, s) mapping; None past the last item."""
    B = len(ctx_lens)
    lane = np.arange(LANES)
    before = 0
    for b0 in range(0, B, LANES):
        ctx = clamp_ctx(ctx_lens, max_ctx, b0)
        f = np.array([chunk_plan(int(c), chunk)[0] for c in ctx])
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
    return None


def expected_order(ctx_lens, max_ctx, chunk):
    ctx = np.clip(np.asarray(ctx_lens), 0, max_ctx)
    return [(b, s) for b in range(len(ctx)) for s in range(chunk_plan(int(ctx[b]), chunk)[0])]


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
def test_items_cover_every_chunk_once_sequence_major(B, chunk, max_ctx, recipe):
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
    # every item maps inside the grid's (sequence, split) range and before the context end; the
    # chunks of a context tile it exactly, none empty, each of chunk/2 .. chunk tokens when the context
    # spans more than one chunk
    ctxc = np.clip(ctx, 0, max_ctx)
    covered = {}
    for b, s in want:
        n, length = chunk_plan(int(ctxc[b]), chunk)
        t0, t1 = s * length, min(int(ctxc[b]), (s + 1) * length)
        assert 0 <= b < B and 0 <= s < nsplit and t0 < t1 <= ctxc[b]
        assert t1 - t0 <= chunk and (n == 1 or 2 * (t1 - t0) >= chunk)
        covered.setdefault(b, []).append((t0, t1))
    for b, spans in covered.items():
        assert spans[0][0] == 0 and spans[-1][1] == ctxc[b]
        assert all(spans[i][1] == spans[i + 1][0] for i in range(len(spans) - 1))


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
