"""GPU parity of mars_accept against the fp64 oracle.

Tokens (argmax) and n_accept are compared bit for bit with the oracle's own outputs; pmax
within 1e-5.  A sequence is left out of the n_accept comparison only when a row that decides
its count (the leading run of rows with pmax >= tau and the first row after it) has an
oracle pmax closer to tau than the measured pmax error (plus tau's fp32 rounding), so that the
two sides may decide it differently; the number left out is asserted (0 on the full workload).
"""
import numpy as np
import pytest
import torch

import structured_mask_attention_amd as M
from oracle import mars_oracle as O
from structured_mask_attention_amd import inputs as I
from tests.gpu_helpers import PMAX_ABS, dev, tie_zone_sequences, tie_zone_width, to_np64

pytestmark = pytest.mark.gpu



def check_accept(logits_cpu, tau, what, ws=None, max_tie=0):
    if logits_cpu.is_contiguous():
        lg = logits_cpu.to(dev())
    else:   # keep the strided layout on the device
        base = logits_cpu
        while base._base is not None:
            base = base._base
        lg = torch.as_strided(base.to(dev()), logits_cpu.shape, logits_cpu.stride(), logits_cpu.storage_offset())
    tok, pmax, n = M.mars_accept(lg, tau, ws=ws)
    torch.cuda.synchronize()
    rtok, rpmax, rn = O.accept(to_np64(logits_cpu), tau)
    tok, pmax, n = tok.cpu().numpy(), pmax.cpu().numpy().astype(np.float64), n.cpu().numpy()
    assert np.array_equal(tok, rtok), f"{what}: argmax differs at {np.argwhere(tok != rtok)[:5]}"
    err = np.abs(pmax - rpmax).max()
    print(f"[{what}] pmax max_abs={err:.3e} n={n.tolist()[:8]}...", flush=True)
    assert err <= PMAX_ABS
    tie = tie_zone_sequences(rpmax, tau, tie_zone_width(pmax, rpmax, tau))
    print(f"[{what}] tie-zone sequences left out of the n_accept comparison: {np.nonzero(tie)[0].tolist()}",
          flush=True)
    assert int(tie.sum()) <= max_tie, f"{what}: {int(tie.sum())} tie-zone sequences (at most {max_tie} expected)"
    assert np.array_equal(n[~tie], rn[~tie]), f"{what}: n_accept differs at {np.nonzero(n != rn)[0].tolist()}"
    return tok, pmax, n


@pytest.mark.parametrize("tau", [0.95, 1.0, 1e-9, 0.5])
def test_accept_full_workload(tau):
    """The full decode workload: no sequence of the seeded draw has a deciding row in the tie
    zone at these thresholds, so every n_accept is compared."""
    s = I.DECODE7B
    logits = I.logits_inputs(s.batch, s.W, s.vocab, seed=s.seed)
    _, pmax, n = check_accept(logits, tau, f"accept 7B tau={tau}", max_tie=0)
    if tau >= 1.0:
        assert (n == 1).all()
    if tau <= 1.0 / s.vocab:
        assert (n == s.W).all()


@pytest.mark.parametrize("tau", [2.0, 0.0, -0.5, float("nan"), float("inf")])
def test_accept_tau_outside_unit_interval_is_rejected(tau):
    """tau must lie in (0, 1]: the call fails before any launch and leaves the outputs alone."""
    s = I.DECODE7B
    lg = I.logits_inputs(2, s.W, 1000, seed=3).to(dev())
    n = torch.full((2,), -7, dtype=torch.int32, device=dev())
    with pytest.raises(M.MarsError) as ei:
        M.mars_accept(lg, tau, n_accept=n)
    assert ei.value.status == -1
    torch.cuda.synchronize()
    assert (n == -7).all()


@pytest.mark.parametrize("batch,W,V", [(3, 4, 1001), (2, 1, 7), (2, 7, 8193), (1, 64, 300), (5, 5, 1), (2, 3, 16384),
                                       (2, 64, 152064)])
def test_accept_shapes(batch, W, V):
    """Ragged vocabularies: rows padded to a 16-byte multiple, the kernel reads V entries."""
    logits = I.logits_inputs(batch, W, V, seed=V + W, spike_hi=8.0)
    Vp = -(-V // 8) * 8
    padded = torch.full((batch, W, Vp), 30.0, dtype=torch.bfloat16)   # pad would win any argmax
    padded[:, :, :V] = logits
    check_accept(padded[:, :, :V], 0.6, f"accept b{batch} W{W} V{V}", max_tie=1)


def test_accept_long_prefixes_at_the_largest_window():
    """Window 64 over the full 152 064-entry vocabulary, each sequence built to stop at a known
    row: rows before k_b carry a spike of 25 (pmax ~ 1 - 1e-5, far above tau = 0.9), row k_b
    none (pmax ~ 1e-5), later rows the spike again, which must not count.  n_accept = k_b, and
    64 when no row is low, with every token and pmax against the oracle."""
    W, V = 64, 152064
    stops = [0, 1, 17, 40, 63, 64]
    x = np.random.default_rng(4711).standard_normal((len(stops), W, V), dtype=np.float32)
    ids = np.random.default_rng(4712).integers(0, V, size=(len(stops), W))
    for bi, k in enumerate(stops):
        for i in range(W):
            if i != k:
                x[bi, i, ids[bi, i]] += 25.0
    tok, _, n = check_accept(I.to_bf16(x), 0.9, "accept long prefixes W64")
    assert n.tolist() == [max(1, k) for k in stops]
    spiked = np.array([[i != k for i in range(W)] for k in stops])
    assert np.array_equal(tok[spiked], ids[spiked])


def test_accept_ties_take_lowest_index():
    V = 20000
    x = torch.zeros((2, 3, V), dtype=torch.bfloat16)
    x[0, 0, [17, 9000, 19999]] = 4.0
    x[0, 1, [15000, 8191, 8192]] = 2.5
    x[0, 2, :] = -1.0
    x[1, 0, [16385, 16384]] = 1.0
    x[1, 1, [0, 1]] = 3.0
    x[1, 2, [19999]] = 3.0
    tok, _, _ = check_accept(x, 0.9, "ties", max_tie=0)
    assert tok.tolist() == [[17, 8191, 0], [16384, 0, 19999]]


def test_accept_workspace_reuse_and_strided_rows():
    """Two calls in a row on one uninitialised workspace, logits as a strided view."""
    s = I.DECODE7B
    big = I.logits_inputs(s.batch, s.W + 1, s.vocab + 64, seed=99)
    view = big[:, 1:, 32:32 + s.vocab]
    ws = torch.full((M.mars_accept_workspace_bytes(s.batch, s.W, s.vocab),), 0x7f, dtype=torch.uint8, device=dev())
    lg = big.to(dev())[:, 1:, 32:32 + s.vocab]
    r1 = M.mars_accept(lg, 0.95, ws=ws)
    r2 = M.mars_accept(lg, 0.95, ws=ws)
    torch.cuda.synchronize()
    for a, b in zip(r1, r2):
        assert torch.equal(a, b)
    rtok, rpmax, _ = O.accept(to_np64(view), 0.95)
    assert np.array_equal(r1[0].cpu().numpy(), rtok)
    assert np.abs(r1[1].cpu().numpy() - rpmax).max() <= PMAX_ABS


def test_accept_extreme_logits():
    """Logits of large magnitude: a row shifted by -30000 (bf16 spacing 128 there, so the top
    entries tie often), a row scaled by 60 (pmax at 1 to fp32 precision or split between
    tied maxima), and a row whose maximum sits in the last vocabulary slice far above the
    rest (the running maximum moves by thousands)."""
    x = I.logits_inputs(2, 4, 152064, 321).float()
    x[0, 0] -= 30000.0
    x[0, 1] *= 60.0
    x[0, 2, -5] = 5000.0
    x[1, 3] = -2.0
    x[1, 3, 17] = 1.0
    for tau in (0.95, 0.5):
        check_accept(x.to(torch.bfloat16), tau, f"extreme logits tau {tau}", max_tie=1)
