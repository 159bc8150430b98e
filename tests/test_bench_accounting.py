"""The benchmark's work counts agree with the oracle's definitions (no GPU)."""
import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("S,window,sinks", [(6, 3, 1), (40, 7, 0), (40, 7, 3), (33, 64, 4), (100, 1, 2)])
def test_window_pair_count_matches_the_oracle_mask(S, window, sinks):
    import bench
    want = int((oracle.window_mask(np.arange(S), S, window, sinks) == 0).sum())  # additive mask: 0 = visible
    assert bench.window_pairs(S, window, sinks) == want
