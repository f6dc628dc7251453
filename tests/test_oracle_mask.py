"""Pins for the oracle's mask and tile map (CPU only).

What fixes the values here, independent of the oracle's own code:
  * the Fig. 2 matrix of the MARS paper (L=8, B=4), hand-derived from §3.2 Eq. 2 and
    stored under tests/golden with its citation;
  * brute-force enumeration of Eq. 2 case by case (loops) against the two-interval
    encoding, over every tiny shape;
  * the nnz closed form (counted per row in plain integers here);
  * Eq. 4 of §3.3 (fraction of masked positions whose context is fully clean = 1/B,
    25% / 12.5% / 6.25% for B = 4 / 8 / 16) and the aitrends.kr summary's ">= 50% AR
    signal with the clean stream";
  * structural statements of §3.2-§3.3 (block 1 sees only the prompt and its own
    earlier masks; causal, not bidirectional, inside a block).
"""
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import mars_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_fig2():
    rows = []
    with open(os.path.join(GOLDEN, "fig2_mask_L8_B4.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append([int(ch) for ch in line])
    return np.array(rows, dtype=np.uint8)


def nnz_closed_form(P, L, B):
    """Visible pairs per head, counted in plain integers (prompt + clean + noisy rows)."""
    prompt = P * (P + 1) // 2
    clean = L * P + L * (L + 1) // 2
    noisy = sum(P + B * (t0 // B) + (t0 % B) + 1 for t0 in range(L))
    return prompt + clean + noisy


def test_fig2_matrix_from_eq2():
    fig2 = load_fig2()
    assert fig2.shape == (16, 16) and int(fig2.sum()) == 72
    assert np.array_equal(O.mask_rules_scalar(0, 8, 4), fig2)
    assert np.array_equal(O.mask_rules(0, 8, 4).astype(np.uint8), fig2)
    assert np.array_equal(O.mask_intervals(0, 8, 4).astype(np.uint8), fig2)


def test_rules_equal_intervals_every_tiny_shape():
    n = 0
    for P in range(0, 5):
        for L in range(0, 13):
            for B in range(1, L + 3):
                if P + 2 * L == 0:
                    continue
                a = O.mask_rules_scalar(P, L, B).astype(bool)
                b = O.mask_intervals(P, L, B)
                c = O.mask_rules(P, L, B)
                assert np.array_equal(a, b), (P, L, B)
                assert np.array_equal(a, c), (P, L, B)
                assert int(a.sum()) == nnz_closed_form(P, L, B) == O.mask_nnz(P, L, B)
                n += 1
    assert n > 400


@settings(max_examples=40, deadline=None)
@given(P=st.integers(0, 40), L=st.integers(1, 60), B=st.integers(1, 70))
def test_rules_equal_intervals_random(P, L, B):
    assert np.array_equal(O.mask_rules(P, L, B), O.mask_intervals(P, L, B))


@pytest.mark.parametrize("P,L,B,expect", [
    (16, 64, 4, 6344),            # tiny fp32 workload
    (256, 512, 4, 557696),        # Qwen2.5-0.5B-shaped layout
    (512, 1536, 8, 4065024),      # Qwen2.5-7B-shaped layout
    (1024, 7168, 32, 66592256),   # long 7B-shaped layout
    (0, 8, 4, 72),                # Fig. 2
])
def test_nnz(P, L, B, expect):
    assert nnz_closed_form(P, L, B) == expect
    assert O.mask_nnz(P, L, B) == expect
    if P + 2 * L <= 4096:
        assert int(O.mask_rules(P, L, B).sum()) == expect


@pytest.mark.parametrize("B,ratio", [(4, 0.25), (8, 0.125), (16, 0.0625)])
def test_eq4_ar_signal_ratio(B, ratio):
    """Eq. 4: only the first position of each block sees a fully clean context."""
    P, L = 5, 64
    m = O.mask_rules(P, L, B)
    noisy = m[P + L:, P + L:]
    only_self = (noisy.sum(axis=1) == 1)
    assert only_self.mean() == ratio
    # the aitrends.kr summary: with the clean stream, >= 50% of positions are AR-like
    assert (L + only_self.sum()) / (2 * L) >= 0.5


def test_first_in_block_sees_exact_ar_context():
    """§3.3: in-block position 1 is conditioned on the clean prefix only (AR-equivalent)."""
    P, L, B = 3, 20, 4
    m = O.mask_rules(P, L, B)
    for k in range(L // B):
        r = P + L + k * B
        expect = np.zeros(P + 2 * L, dtype=bool)
        expect[:P + k * B] = True
        expect[r] = True
        assert np.array_equal(m[r], expect)


def test_block1_sees_prompt_and_own_masks_only():
    P, L, B = 6, 16, 4
    m = O.mask_rules(P, L, B)
    for t in range(B):
        r = P + L + t
        seen = set(np.nonzero(m[r])[0].tolist())
        assert seen == set(range(P)) | set(range(P + L, r + 1))


def test_causal_not_bidirectional_inside_block():
    P, L, B = 2, 12, 4
    m = O.mask_rules(P, L, B)
    for k in range(L // B):
        blk = m[P + L + k * B:P + L + (k + 1) * B, P + L + k * B:P + L + (k + 1) * B]
        assert np.array_equal(blk, np.tril(np.ones((B, B), dtype=bool)))


def test_prompt_and_clean_rows_are_plain_causal():
    P, L, B = 7, 9, 2
    m = O.mask_rules(P, L, B)
    n = P + L
    assert np.array_equal(m[:n, :n], np.tril(np.ones((n, n), dtype=bool)))
    assert not m[:n, n:].any()


def test_every_row_sees_itself():
    for (P, L, B) in [(0, 5, 3), (4, 9, 9), (3, 7, 1), (1, 6, 10)]:
        m = O.mask_rules(P, L, B)
        assert m[np.arange(P + 2 * L), np.arange(P + 2 * L)].all()


# ---- tile map -------------------------------------------------------------

@pytest.mark.parametrize("P,L,B,counts", [
    (16, 64, 4, (1, 3, 0)),
    (256, 512, 4, (57, 14, 29)),
    (512, 1536, 8, (510, 40, 234)),
])
def test_tile_counts_128(P, L, B, counts):
    tm = O.tile_map_rules(P, L, B, 128, 128)
    got = (int((tm == 0).sum()), int((tm == 1).sum()), int((tm == 2).sum()))
    assert got == counts


@pytest.mark.slow
def test_tile_counts_128_long():
    tm = O.tile_map_rules(1024, 7168, 32, 128, 128)
    assert (int((tm == 0).sum()), int((tm == 1).sum()), int((tm == 2).sum())) == (10220, 176, 4004)


def test_tile_map_brute_force_tiny():
    """Class of each tile by direct enumeration of its elements with the loop rules."""
    for (P, L, B, bm, bn) in [(3, 10, 3, 4, 5), (0, 8, 4, 4, 4), (5, 11, 2, 7, 3), (2, 9, 12, 16, 16)]:
        m = O.mask_rules_scalar(P, L, B)
        N = P + 2 * L
        tm = O.tile_map_rules(P, L, B, bm, bn)
        for a in range(tm.shape[0]):
            for c in range(tm.shape[1]):
                vals = [m[i, j] for i in range(a * bm, min(N, a * bm + bm))
                        for j in range(c * bn, min(N, c * bn + bn))]
                expect = 2 if all(vals) else (1 if any(vals) else 0)
                assert tm[a, c] == expect


@pytest.mark.parametrize("P,L,B,flop_vt", [
    (256, 512, 4, 2.020e10 / (8 * 14 * 4 * 64)),
    (512, 1536, 8, 2.574e11 / (4 * 28 * 4 * 128)),
])
def test_visible_tile_elems(P, L, B, flop_vt):
    e = O.visible_tile_elems(P, L, B, 128, 128)
    assert abs(e - flop_vt) / flop_vt < 2e-3
    assert e >= O.mask_nnz(P, L, B)
