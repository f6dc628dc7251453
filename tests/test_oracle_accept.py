"""Pins for the oracle's acceptance rule (CPU only).

Anchors: the MARS blog ("commits them left to right while its confidence holds,
stopping at the first token below a threshold tau"; "tau=1.0 recovers exact
single-token AR decoding"), the aitrends.kr summary (at least one token is always
accepted), greedy decoding (argmax), and closed forms of the softmax maximum.
"""
import math

import numpy as np
import pytest
import torch

from oracle import mars_oracle as O


def test_tau_one_is_exact_ar():
    x = np.zeros((3, 4, 50))
    x[:, :, 7] = 200.0                      # pmax rounds to 1.0 in float64
    tok, pmax, n = O.accept(x, 1.0)
    assert (pmax == 1.0).all() and (n == 1).all() and (tok == 7).all()


def test_tau_below_uniform_accepts_whole_window():
    x = np.random.default_rng(1).standard_normal((4, 5, 33))
    _, pmax, n = O.accept(x, 1.0 / 33)
    assert (pmax >= 1.0 / 33).all() and (n == 5).all()


def test_constant_row():
    _, pmax, _ = O.accept(np.full((1, 1, 1000), -3.25), 0.5)
    tok, _, _ = O.accept(np.full((1, 1, 1000), -3.25), 0.5)
    assert pmax[0, 0] == 1.0 / 1000 and tok[0, 0] == 0


@pytest.mark.parametrize("h,V", [(0.0, 10), (2.5, 100), (20.0, 152064), (-4.0, 7)])
def test_single_spike_closed_form(h, V):
    x = np.zeros((1, 1, V))
    x[0, 0, V // 3] = h
    tok, pmax, _ = O.accept(x, 0.5)
    if h >= 0:   # the spike is the maximum (ties at h = 0 go to index 0)
        expect = math.exp(h) / (math.exp(h) + V - 1)
        expect_tok = V // 3 if h > 0 else 0
    else:        # the zeros are the maximum
        expect = 1.0 / (V - 1 + math.exp(h))
        expect_tok = 0
    assert abs(pmax[0, 0] - expect) <= 1e-15 * max(1.0, expect)
    assert tok[0, 0] == expect_tok


def test_ties_take_lowest_index():
    x = np.zeros((1, 2, 9))
    x[0, 0, [3, 5]] = 4.0
    x[0, 1, [8, 2, 6]] = 1.5
    tok, _, _ = O.accept(x, 0.9)
    assert tok.tolist() == [[3, 2]]


def test_prefix_stops_at_first_below_tau():
    def row(p, V=10):
        # logits giving top-1 probability p: one entry log(p (V-1) / (1 - p)), others 0
        r = np.zeros(V)
        r[0] = math.log(p * (V - 1) / (1 - p))
        return r
    x = np.stack([np.stack([row(0.99), row(0.5), row(0.99), row(0.99)]),
                  np.stack([row(0.99), row(0.99), row(0.2), row(0.99)]),
                  np.stack([row(0.1), row(0.99), row(0.99), row(0.99)]),
                  np.stack([row(0.97), row(0.96), row(0.99), row(0.951)])])
    _, pmax, n = O.accept(x, 0.95)
    assert n.tolist() == [1, 2, 1, 4]
    _, _, n2 = O.accept(x, 0.995)
    assert n2.tolist() == [1, 1, 1, 1]


def test_matches_scalar_and_torch_softmax():
    x = np.random.default_rng(2).standard_normal((3, 4, 257)) * 3
    x[1, 2, 17] += 15
    tok, pmax, n = O.accept(x, 0.6)
    tok2, pmax2, n2 = O.accept_scalar(x, 0.6)
    assert np.array_equal(tok, tok2) and np.array_equal(n, n2)
    assert np.max(np.abs(pmax - pmax2)) <= 1e-15
    sm = torch.softmax(torch.from_numpy(x), -1)
    assert np.max(np.abs(sm.max(-1).values.numpy() - pmax)) <= 1e-15
    assert np.array_equal(sm.argmax(-1).numpy(), tok)


# ---------------------------------------------------------------------------
# Margin gate (top-1 minus top-2 probability)
# ---------------------------------------------------------------------------

def test_margin_matches_scalar_brute_force():
    rng = np.random.default_rng(71)
    for V in (2, 3, 7, 33):
        x = np.round(rng.standard_normal((3, 4, V)) * 2, 1)   # coarse values: ties happen
        t, pm, mg, n = O.accept_margin(x, 0.3)
        t2, mg2, n2 = O.accept_margin_scalar(x, 0.3)
        assert np.array_equal(t, t2) and np.array_equal(n, n2)
        assert np.max(np.abs(mg - mg2)) < 1e-12
        # brute force: sort the probabilities
        p = np.exp(x - x.max(axis=-1, keepdims=True))
        p /= p.sum(axis=-1, keepdims=True)
        ps = np.sort(p, axis=-1)
        assert np.max(np.abs(mg - (ps[..., -1] - ps[..., -2]))) < 1e-12


def test_margin_closed_forms():
    V = 1000
    # one spike of height h over zeros: p1 = e^h / (e^h + V - 1), p2 = 1 / (e^h + V - 1)
    for h in (0.5, 3.0, 12.0):
        x = np.zeros((1, 1, V))
        x[0, 0, 17] = h
        t, pm, mg, n = O.accept_margin(x, 0.5)
        den = math.exp(h) + V - 1
        assert t[0, 0] == 17 and abs(mg[0, 0] - (math.exp(h) - 1) / den) < 1e-12
    # a tied maximum (two equal top entries) has margin exactly 0; a constant row too
    x = np.zeros((1, 2, V))
    x[0, 0, [5, 9]] = 4.0
    t, pm, mg, n = O.accept_margin(x, 1e-9)
    assert mg[0, 0] == 0.0 and mg[0, 1] == 0.0 and t[0, 0] == 5 and n[0] == 1
    # a one-entry vocabulary has no second entry: margin = top-1 probability = 1
    t, pm, mg, n = O.accept_margin(np.full((1, 3, 1), 2.0), 0.999)
    assert np.all(mg == 1.0) and np.all(t == 0) and n[0] == 3
    t2, mg2, n2 = O.accept_margin_scalar(np.full((1, 3, 1), 2.0), 0.999)
    assert np.all(mg2 == 1.0) and n2[0] == 3


def test_margin_gate_prefix_and_tau_one():
    V = 50
    x = np.zeros((2, 4, V))
    for i, h in enumerate((30.0, 30.0, 0.1, 30.0)):   # margins ~1, ~1, small, ~1
        x[:, i, 3] = h
    _, _, mg, n = O.accept_margin(x, 0.9)
    assert list(n) == [2, 2]                           # stops at the first small margin
    _, _, _, n1 = O.accept_margin(x, 1.0)
    assert list(n1) == [1, 1]                          # exact AR fallback
    _, _, _, n0 = O.accept_margin(x, 1e-12)
    assert list(n0) == [4, 4]                          # every margin is > 0 here
