"""CPU pins of the GPU tests' own expectations (test infrastructure built on the oracle)."""
import itertools

import numpy as np

from tests.gpu_helpers import expected_tilelog, expected_tilelog_intervals, tie_zone_sequences


def test_tilelog_expectation_encodings_agree():
    """The interval-based expected tile log (used at full size) equals the one read off the
    oracle's dense Eq. 2 mask on every small shape, ragged tiles, P = 0, L = 0, B = 1 and
    B > L included."""
    for P, L, B, G in itertools.product([0, 3, 40], [0, 1, 5, 37, 70], [1, 3, 8, 32], [1, 2, 7]):
        if P + 2 * L == 0:
            continue
        for rb, kb in ((32, 32), (16, 48)):
            assert np.array_equal(expected_tilelog(P, L, B, G, rb, kb), expected_tilelog_intervals(P, L, B, G, rb, kb)), \
                (P, L, B, G, rb, kb)


def test_tie_zone_only_counts_deciding_rows():
    g = np.array([[0.99, 0.96, 0.9500001, 0.2],     # row 2 is in the run but not in the zone (width 1e-8)
                  [0.99, 0.2, 0.9500001, 0.99],     # row 2 comes after the first row below tau
                  [0.9500001, 0.1, 0.1, 0.1],       # the deciding row 0 is in the zone
                  [0.2, 0.95000001, 0.1, 0.1]])     # row 0 decides (below tau); row 1 does not count
    assert tie_zone_sequences(g, 0.95, 1e-8).tolist() == [False, False, False, False]
    assert tie_zone_sequences(g, 0.95, 1e-6).tolist() == [True, False, True, False]
    assert not tie_zone_sequences(g, 1.0, 1.0).any()
