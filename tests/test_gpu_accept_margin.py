"""GPU parity of mars_accept_margin (the margin gate) against the fp64 oracle.

Tokens and n_accept bit for bit with the oracle's own outputs, margin and pmax within 1e-5.  A
sequence is left out of the n_accept comparison only when a row that decides its count (the
leading run of rows with margin >= tau and the first row after it) has an oracle margin closer to
tau than the measured margin error (plus tau's fp32 rounding), so that the two sides may decide it
differently; the number left out is asserted (0 on the full workload).
"""
import numpy as np
import pytest
import torch

import structured_mask_attention_amd as M
from oracle import mars_oracle as O
from structured_mask_attention_amd import inputs as I
from tests.gpu_helpers import PMAX_ABS, dev, tie_zone_sequences, tie_zone_width, to_np64

pytestmark = pytest.mark.gpu



def check_margin(logits_cpu, tau, what, max_tie=0):
    if logits_cpu.is_contiguous():
        lg = logits_cpu.to(dev())
    else:   # keep the strided (row-padded) layout on the device
        base = logits_cpu
        while base._base is not None:
            base = base._base
        lg = torch.as_strided(base.to(dev()), logits_cpu.shape, logits_cpu.stride(), logits_cpu.storage_offset())
    tok, pmax, mg, n = M.mars_accept_margin(lg, tau)
    torch.cuda.synchronize()
    rtok, rpmax, rmg, rn = O.accept_margin(to_np64(logits_cpu), tau)
    tok, pmax, mg, n = (t.cpu().numpy() for t in (tok, pmax, mg, n))
    assert np.array_equal(tok, rtok), f"{what}: argmax differs at {np.argwhere(tok != rtok)[:5]}"
    e_m = np.abs(mg.astype(np.float64) - rmg).max()
    e_p = np.abs(pmax.astype(np.float64) - rpmax).max()
    print(f"[{what}] margin max_abs={e_m:.3e} pmax max_abs={e_p:.3e} n={n.tolist()[:8]}...", flush=True)
    assert e_m <= PMAX_ABS and e_p <= PMAX_ABS
    # A tied maximum gives margin exactly 0 on both sides (the kernel forms 1 - exp(0) = 0), so
    # those rows are decided exactly: they never count as tie-zone rows.
    tie = tie_zone_sequences(np.where(rmg == 0.0, -np.inf, rmg), tau, tie_zone_width(mg, rmg, tau))
    print(f"[{what}] tie-zone sequences left out of the n_accept comparison: {np.nonzero(tie)[0].tolist()}",
          flush=True)
    assert int(tie.sum()) <= max_tie, f"{what}: {int(tie.sum())} tie-zone sequences (at most {max_tie} expected)"
    assert np.array_equal(n[~tie], rn[~tie]), f"{what}: n_accept differs at {np.nonzero(n != rn)[0].tolist()}"
    return tok, mg, n


@pytest.mark.parametrize("tau", [0.3, 0.9, 1.0, 1e-9])
def test_margin_full_workload(tau):
    s = I.DECODE7B
    logits = I.logits_inputs(s.batch, s.W, s.vocab, seed=s.seed)
    _, mg, n = check_margin(logits, tau, f"margin 7B tau={tau}")
    if tau >= 1.0:
        assert (n == 1).all()


@pytest.mark.parametrize("batch,W,V", [(3, 4, 1001), (2, 1, 7), (2, 7, 8193), (1, 64, 300), (5, 5, 1), (2, 3, 16384),
                                       (2, 2, 40000), (2, 64, 152064)])
def test_margin_shapes(batch, W, V):
    """Ragged vocabularies: rows padded to a 16-byte multiple, the kernel reads V entries."""
    logits = I.logits_inputs(batch, W, V, seed=V + 3 * W, spike_hi=8.0)
    Vp = -(-V // 8) * 8
    padded = torch.full((batch, W, Vp), 30.0, dtype=torch.bfloat16)   # pad would win any max
    padded[:, :, :V] = logits
    check_margin(padded[:, :, :V], 0.4, f"margin b{batch} W{W} V{V}", max_tie=1)


def test_margin_top_two_across_slices_and_ties():
    """The two largest entries in different 16384-entry slices, equal or not; a tied maximum
    gives margin 0 exactly."""
    V = 40000
    x = torch.full((2, 4, V), -2.0, dtype=torch.bfloat16)
    x[0, 0, [3, 39000]] = 5.0                 # tied maximum in the first and last slice
    x[0, 1, 20000] = 5.0
    x[0, 1, 100] = 4.5                        # second largest in another slice
    x[0, 2, 16383] = 3.0
    x[0, 2, 16384] = 3.0                      # tie across the slice boundary
    x[0, 3, 7] = 6.0                          # single spike
    x[1, :, :] = 0.0                          # constant rows: margin 0
    tok, mg, _ = check_margin(x, 0.1, "top-2 across slices")
    assert mg[0, 0] == 0.0 and mg[0, 2] == 0.0 and np.all(mg[1] == 0.0)
    assert tok[0].tolist() == [3, 20000, 16383, 7]


def test_margin_extreme_logits():
    x = I.logits_inputs(2, 4, 152064, 321).float()
    x[0, 0] -= 30000.0
    x[0, 1] *= 60.0
    x[0, 2, -5] = 5000.0
    x[1, 3] = -2.0
    x[1, 3, 17] = 1.0
    check_margin(x.to(torch.bfloat16), 0.3, "margin extreme logits", max_tie=1)
