"""Host model of the fused RoPE table + K rotation pass (csrc/rope.hip, rope_table_rotate_bf16_kernel).

A work-group of 256 threads covers the items first .. first+255 of (s, g, 8-pair group), i.e. the
positions p0 .. p1, and stages those positions' (cos, sin) entries in an LDS array of fixed size.
The checks replay the kernel's index arithmetic on the CPU for every work-group and prove that the
staged entries fit the array, that every thread reads entries it staged (and of its own position),
and that the work-groups together write every table entry. No GPU is needed.
"""
import numpy as np
import pytest

MAX_D = 512               # kTableRotMaxD: larger head dims take the two-launch form
LDS_ENTRIES = 2040 + MAX_D  # kTableRotLds


@pytest.mark.parametrize("S,N,D", [(8192, 8, 128), (1024, 12, 64), (333, 1, 128), (77, 5, 16), (129, 3, 512),
                                   (50, 1, 512), (1, 1, 16), (4096, 32, 64)])
def test_staged_entries_fit_and_cover_every_read(S, N, D):
    assert D % 16 == 0 and D <= MAX_D
    half, groups = D // 2, D // 16
    total = S * N * groups
    written = np.zeros(S * half, dtype=bool)
    for blk in range((total + 255) // 256):
        first = blk * 256
        last = min(first + 255, total - 1)
        p0, p1 = first // groups // N, last // groups // N
        nent = (p1 - p0 + 1) * half
        assert nent <= LDS_ENTRIES
        e = np.arange(nent)
        pos, i = p0 + e // half, e % half
        assert pos.max() < S
        written[pos * half + i] = True
        idx = np.arange(first, last + 1)
        i0 = (idx % groups) * 8
        p = (idx // groups) // N
        lo = (p - p0) * half + i0
        assert lo.min() >= 0 and (lo + 7).max() < nent
        # the staged entry at lo + e is (p, i0 + e): same position, same pair index
        assert np.all(p0 + lo // half == p) and np.all((lo % half) == i0)
    assert written.all()


def test_lds_bound_is_tight_for_the_largest_head_dim():
    """The bound (255 // (N * D/16) + 2) * D/2 <= 2040 + D, reached for N = 1."""
    worst = 0
    for D in range(16, MAX_D + 1, 16):
        for N in (1, 2, 3, 7, 8):
            worst = max(worst, (255 // (N * (D // 16)) + 2) * (D // 2))
    assert worst <= LDS_ENTRIES


@pytest.mark.parametrize("D,roff,Dr", [(192, 128, 64), (576, 512, 64), (128, 0, 128), (64, 32, 32)])
def test_span_pass_writes_every_element_once(D, roff, Dr):
    """The k^R span pass: per row, roff/8 threads copy 8 dims, Dr/16 threads rotate 8 pairs (i, i + Dr/2)
    each; together they write every element of the row once, and a rotating thread reads exactly the
    two 8-element halves it writes."""
    ncopy, nrot, half = roff // 8, Dr // 16, Dr // 2
    written = []
    for gi in range(ncopy + nrot):
        if gi < ncopy:
            written += list(range(8 * gi, 8 * gi + 8))
        else:
            i0 = 8 * (gi - ncopy)
            assert i0 + 8 <= half
            written += list(range(roff + i0, roff + i0 + 8)) + list(range(roff + half + i0, roff + half + i0 + 8))
    assert roff + Dr == D  # the launcher's precondition: the span ends the row
    assert sorted(written) == list(range(D))
