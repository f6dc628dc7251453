"""GPU parity of mars_shifted_ce (L_mask, L_AR and their logits gradient) against the
fp64 oracle.

Bounds, from the kernel's arithmetic (bf16 logits are exact inputs; everything after is
fp32 with one bf16 rounding of the gradient):
  * per-row CE, computed as (fma(x_t, -log2 e, c) + log2 S) ln 2 with c = fl(max log2 e)
    and S the sum of exp2(fma(x, log2 e, -c)): the sum carries at most ~200 fp32
    additions per thread and a 16-way merge (relative 2e-5, so 5e-5 nats with the log);
    every other rounding is relative to the CE itself (the fma's exact product removes
    the magnitude of the logits), so ROW_CE = 5e-5 + 1e-6 |CE| nats;
  * losses: the sum of their rows' ROW_CE, plus n 2^-24 of sum |CE| for the fp32 sum;
  * gradient entries w (p - onehot), p = exp2(fma(x, log2 e, -lse2)) with lse2 = c +
    log2 S rounded once at its own magnitude: the exponent is off by at most 1e-4 +
    1.2e-7 |lse| nats (the sum as above, and 2^-24 |lse2| ln 2 with a factor 2 margin), so
    p is within that relative error (plus 2^-22 for exp2), and the result is rounded once
    to bf16 (2^-8 of the value).
"""
import numpy as np
import pytest
import torch

import structured_mask_attention_amd as M
from oracle import mars_oracle as O
from structured_mask_attention_amd import inputs as I
from tests.gpu_helpers import dev, to_np64

pytestmark = pytest.mark.gpu


def row_terms(z, x, P, L, B):
    """Per (sequence, row): the oracle's lse, CE and ROW bound (0 where no target), and the
    targets and weights."""
    tgt, war, wmask = O.shifted_ce_targets(P, L, B)
    zz = np.asarray(z, dtype=np.float64)
    m = zz.max(axis=-1, keepdims=True)
    lse = m[..., 0] + np.log(np.exp(zz - m).sum(axis=-1))
    b = zz.shape[0]
    ce = np.zeros((b, len(tgt)))
    rb = np.zeros((b, len(tgt)))
    has = tgt >= 0
    for bi in range(b):
        xt = zz[bi, has, x[bi, tgt[has]]]
        ce[bi, has] = lse[bi, has] - xt
        rb[bi, has] = 5e-5 + 1e-6 * np.abs(ce[bi, has])
    return lse, ce, rb, tgt, war, wmask


def check_losses(lm, la, ref_lm, ref_la, z, x, P, L, B, what):
    _, ce, rb, tgt, war, wmask = row_terms(z, x, P, L, B)
    for bi in range(z.shape[0]):
        for name, got, ref, w in (("L_mask", lm, ref_lm, wmask), ("L_AR", la, ref_la, war)):
            err = abs(float(got[bi]) - ref[bi])
            n = np.count_nonzero(w)
            bound = (w * rb[bi]).sum() + n * 2.0 ** -24 * np.abs(w * ce[bi]).sum() + 1e-6
            print(f"[{what} b{bi} {name}] got={float(got[bi]):.6f} ref={ref[bi]:.6f} err={err:.2e} bound={bound:.2e}", flush=True)
            assert np.isfinite(got[bi]) and err <= bound, f"{what}: {name} of sequence {bi} off by {err}"


def check_grad(got, ref, z, x, P, L, B, what, rows=None):
    """``got``/``ref`` hold the rows ``rows`` (all rows if None) of the gradient."""
    lse, _, _, tgt, war, wmask = row_terms(z, x, P, L, B)
    w = war + wmask
    if rows is not None:
        tgt, w, lse = tgt[rows], w[rows], lse[:, rows]
        zr = np.asarray(z, dtype=np.float64)[:, rows]
    else:
        zr = np.asarray(z, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite gradient"
    p = np.exp(zr - lse[..., None])                            # the oracle's softmax
    rel_p = 1e-4 + 1.2e-7 * np.abs(lse) + 2.0 ** -22                # [b, rows]
    bound = 2.0 ** -8 * np.abs(ref) + w[None, :, None] * p * rel_p[..., None] * 1.01 + 1e-37
    err = np.abs(got - ref)
    ratio = float(np.max(err / bound)) if err.size else 0.0
    print(f"[{what} dlogits] max_abs={float(err.max()) if err.size else 0:.3e} max err/bound={ratio:.3f}", flush=True)
    assert ratio <= 1.0, f"{what}: gradient error exceeds its bound (ratio {ratio:.3f})"
    # rows that predict nothing are exactly zero
    for k, t in enumerate(tgt):
        if t < 0:
            assert np.all(got[:, k] == 0.0), f"{what}: row {k} without a target has a nonzero gradient"


def run_case(b, P, L, B, V, seed, what):
    print(f"case shifted_ce {what} b={b} P={P} L={L} B={B} V={V} seed={seed}", flush=True)
    logits, tokens = I.ce_inputs(b, P, L, V, seed)
    z, x = to_np64(logits), tokens.numpy().astype(np.int64)
    lm, la, dl = M.mars_shifted_ce(logits.to(dev()), tokens.to(dev()), P, L, B, grad=True)
    torch.cuda.synchronize()
    ref_lm, ref_la, ref_d = O.shifted_ce(z, x, P, L, B)
    check_losses(to_np64(lm), to_np64(la), ref_lm, ref_la, z, x, P, L, B, what)
    check_grad(to_np64(dl), ref_d, z, x, P, L, B, what)
    return lm, la, dl


@pytest.mark.parametrize("b,P,L,B,V", [
    (2, 5, 12, 4, 1000),            # ragged last vector slice (1000 / 8 = 125 vectors)
    (1, 0, 9, 4, 64),               # no prompt: x_0 has no AR term
    (2, 3, 6, 1, 256),              # B = 1: every token is a block start
    (1, 4, 3, 8, 512),              # B > L
    (1, 7, 1, 4, 72),               # L = 1: no noisy row predicts anything
    (1, 6, 0, 4, 128),              # prompt only: both losses 0, gradient all zero
    (1, 2, 5, 2, 8),                # smallest vocabulary (one vector)
    (2, 64, 128, 4, 4096),          # several blocks, V of 4 vectors per thread
    (1, 3, 10, 4, 8 * 1024 + 8),    # two vectors per thread, second one mostly padding
    (1, 2, 6, 4, 8 * 1024 * 20),    # largest register-resident vocabulary
    (1, 2, 6, 4, 8 * 1024 * 20 + 8),   # streaming kernel (vocabulary beyond registers)
    (1, 1, 5, 2, 262144),           # streaming kernel, larger vocabulary
])
def test_ce_small_all_elements(b, P, L, B, V):
    run_case(b, P, L, B, V, 31 + V + 7 * L, f"P{P} L{L} B{B} V{V}")


def test_ce_loss_only_matches_gradient_run_bitwise():
    b, P, L, B, V = 2, 16, 40, 4, 151936
    logits, tokens = I.ce_inputs(b, P, L, V, 5, device=dev())
    a = M.mars_shifted_ce(logits, tokens, P, L, B, grad=True)
    c = M.mars_shifted_ce(logits, tokens, P, L, B, grad=False)
    d = M.mars_shifted_ce(logits, tokens, P, L, B, grad=True)
    torch.cuda.synchronize()
    assert c[2] is None
    assert torch.equal(a[0], c[0]) and torch.equal(a[1], c[1])
    assert torch.equal(a[0], d[0]) and torch.equal(a[1], d[1]) and torch.equal(a[2], d[2])


def test_ce_strided_views():
    """Logits and the gradient as row-strided views of wider buffers; padding untouched."""
    b, P, L, B, V = 2, 4, 10, 4, 512
    N = P + 2 * L
    logits, tokens = I.ce_inputs(b, P, L, V, 11)
    big = torch.zeros((b, N, V + 64), dtype=torch.bfloat16)
    big[..., :V] = logits
    lv = big.to(dev())[..., :V]
    tok_big = torch.zeros((b, L + 3), dtype=torch.int32)
    tok_big[:, :L] = tokens
    tv = tok_big.to(dev())[:, :L]
    dbuf = torch.full((b, N, V + 32), 3.0, dtype=torch.bfloat16, device=dev())
    dv = dbuf[..., :V]
    lm, la, _ = M.mars_shifted_ce(lv, tv, P, L, B, grad=True, dlogits=dv)
    ref = M.mars_shifted_ce(logits.to(dev()), tokens.to(dev()), P, L, B, grad=True)
    torch.cuda.synchronize()
    assert torch.equal(lm, ref[0]) and torch.equal(la, ref[1]) and torch.equal(dv, ref[2])
    assert torch.all(dbuf[..., V:] == 3.0)


def test_ce_full_size_qwen05b():
    """The training workload's loss: Qwen2.5-0.5B layout [8, 1280] rows over its 151936-entry
    vocabulary, in the launch the bench times.  Sequence 0 is checked whole against the
    oracle (both losses, the gradient on sampled rows); every sequence's losses are finite
    and non-negative."""
    s = I.QWEN05B
    V = 151936
    print(f"case shifted_ce full size {s.name} V={V}", flush=True)
    logits, tokens = I.ce_inputs(s.batch, s.P, s.L, V, 2002, device=dev())
    lm, la, dl = M.mars_shifted_ce(logits, tokens, s.P, s.L, s.B, grad=True)
    torch.cuda.synchronize()
    assert torch.isfinite(lm).all() and torch.isfinite(la).all()
    assert (lm >= 0).all() and (la >= 0).all()
    z = to_np64(logits[:1])
    x = tokens[:1].cpu().numpy().astype(np.int64)
    ref_lm, ref_la, ref_d = O.shifted_ce(z, x, s.P, s.L, s.B)
    check_losses(to_np64(lm[:1]), to_np64(la[:1]), ref_lm, ref_la, z, x, s.P, s.L, s.B, "qwen0.5b")
    rows = np.unique(np.concatenate([[0, s.P - 2, s.P - 1, s.P, s.P + s.L - 1, s.P + s.L, s.N - 2, s.N - 1],
                                     np.random.default_rng(3).integers(0, s.N, 24)]))
    check_grad(to_np64(dl[:1, rows]), ref_d[:, rows], z, x, s.P, s.L, s.B, "qwen0.5b", rows=rows)


def test_ce_extreme_and_constant_rows():
    """Rows whose maximum first appears in a late vector at a large value (the running offset
    must move by thousands of nats), rows of equal entries (CE = ln V exactly in exact
    arithmetic) and large negative rows, on the register-resident kernel (V = 151936) and
    the streaming one (V = 200000)."""
    for V in (151936, 200000):
        b, P, L, B = 1, 2, 6, 4
        N = P + 2 * L
        logits, tokens = I.ce_inputs(b, P, L, V, 77)
        z = logits.float().clone()
        z[0, 4] = 0.0                                   # constant row (predicts x_3)
        z[0, 1, -3] = 3000.0                            # maximum in the last vector, far above the rest
        z[0, 2] = z[0, 2] - 5000.0                      # large negative row
        z[0, 3, :] = -2.0
        z[0, 3, V // 2] = 40.0                          # one dominant entry mid-row
        logits = z.to(torch.bfloat16)
        tokens[0, 0] = V - 3                            # row P - 1 = 1 predicts the spiked entry
        run = M.mars_shifted_ce(logits.to(dev()), tokens.to(dev()), P, L, B, grad=True)
        torch.cuda.synchronize()
        zz, x = to_np64(logits), tokens.numpy().astype(np.int64)
        ref_lm, ref_la, ref_d = O.shifted_ce(zz, x, P, L, B)
        check_losses(to_np64(run[0]), to_np64(run[1]), ref_lm, ref_la, zz, x, P, L, B, f"extreme V{V}")
        check_grad(to_np64(run[2]), ref_d, zz, x, P, L, B, f"extreme V{V}")


def test_ce_out_of_range_tokens_give_infinite_loss():
    """Tokens outside [0, V) are compared, never used as an index: the terms they enter
    are +inf, the other sequence's losses and every gradient stay finite."""
    for V in (4096, 200000):
        b, P, L, B = 2, 3, 5, 4
        logits, tokens = I.ce_inputs(b, P, L, V, 13)
        tokens[0, 1] = V
        tokens[0, 2] = -1
        lm, la, dl = M.mars_shifted_ce(logits.to(dev()), tokens.to(dev()), P, L, B, grad=True)
        torch.cuda.synchronize()
        assert torch.isinf(la[0]) and la[0] > 0 and torch.isinf(lm[0]) and lm[0] > 0
        ref_lm, ref_la, _ = O.shifted_ce(to_np64(logits[1:]), tokens[1:].numpy().astype(np.int64), P, L, B)
        assert abs(float(la[1]) - ref_la[0]) < 1e-3 and abs(float(lm[1]) - ref_lm[0]) < 1e-3
        assert torch.isfinite(dl).all()
