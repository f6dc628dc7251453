"""Seeded random-shape sweep of every hot-path kernel against the fp64 oracle (whole outputs).

The shapes are drawn once from a fixed NumPy generator (seed 20261202), so every run checks
the same cases; each case prints its shape before it runs.  Training-layout forward: batch,
GQA group, KV heads, head_dim, prompt, response and block length (MARS §3.2 Eq. 2), with the
visited-tile log checked bit for bit; backward on the same kind of shapes and on five
mid-size ones (about 1000-4000 positions, so the dK/dV walks split into chunks); decode step: batch,
group, KV heads, head_dim, window, cache capacity and per-sequence lengths (0 and the capacity
included; MARS Fig. 2 right); acceptance: batch, window, vocabulary and tau (the MARS author
blog, "Inference: a knob, not a mode switch").
"""
import numpy as np
import pytest
import torch

import structured_mask_attention_amd as M
from oracle import mars_oracle as O
from structured_mask_attention_amd import inputs as I
from tests.gpu_helpers import (LSE_FIXED, PMAX_ABS, bwd_bounds, check_bounded, check_close, dev,
                               expected_tilelog_intervals, lse_bound, tie_zone_sequences, tie_zone_width, to_np64)

pytestmark = pytest.mark.gpu

_RNG = np.random.default_rng(20261202)


def _train_shapes(n, max_pl):
    out = []
    for _ in range(n):
        G = int(_RNG.choice([1, 2, 3, 4, 7]))
        hkv = int(_RNG.integers(1, 4))
        d = int(_RNG.choice([64, 128]))
        P = int(_RNG.integers(0, max_pl))
        L = int(_RNG.integers(0, max_pl))
        if P + 2 * L == 0:
            L = 1
        B = int(_RNG.choice([1, 2, 3, 4, 5, 8, 16, 32, 40]))
        b = int(_RNG.integers(1, 3))
        out.append((b, G * hkv, hkv, d, P, L, B, int(_RNG.integers(0, 1 << 30))))
    return out


FWD_SHAPES = _train_shapes(16, 160)
BWD_SHAPES = _train_shapes(6, 90)


def _decode_shapes(n):
    out = []
    for _ in range(n):
        G = int(_RNG.choice([1, 2, 4, 7, 8]))
        W = int(_RNG.integers(1, 64 // G + 1))
        hkv = int(_RNG.integers(1, 4))
        d = int(_RNG.choice([64, 128]))
        cap = int(_RNG.choice([0, 1, 31, 512, 513, 1500]))
        batch = int(_RNG.integers(1, 6))
        lens = _RNG.integers(0, cap + 1, size=batch)
        if batch >= 2:
            lens[0], lens[-1] = 0, cap
        out.append((batch, G * hkv, hkv, d, W, cap, lens.tolist(), int(_RNG.integers(0, 1 << 30))))
    return out


DEC_SHAPES = _decode_shapes(8)


def _accept_shapes(n):
    out = []
    for _ in range(n):
        batch = int(_RNG.integers(1, 9))
        W = int(_RNG.integers(1, 17))
        V = int(_RNG.choice([1, 2, 9, 1000, 16385, 70001, 152064]))
        tau = float(_RNG.choice([1.0, 0.95, 0.5, 0.1, 1e-6]))
        out.append((batch, W, V, tau, int(_RNG.integers(0, 1 << 30))))
    return out


ACC_SHAPES = _accept_shapes(8)


@pytest.mark.parametrize("b,hq,hkv,d,P,L,B,seed", FWD_SHAPES)
def test_sweep_forward(b, hq, hkv, d, P, L, B, seed):
    print(f"case sweep fwd b={b} hq={hq} hkv={hkv} d={d} P={P} L={L} B={B} seed={seed}", flush=True)
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, seed)
    N = P + 2 * L
    qd, kd, vd = q.to(dev()), k.to(dev()), v.to(dev())
    lse = torch.empty((b, hq, N), dtype=torch.float32, device=dev())
    out, log = M.mars_attn_fwd_tilelog(qd, kd, vd, P, L, B, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = O.attn(to_np64(q), to_np64(k), to_np64(v), P, L, B)
    check_close(to_np64(out), ref, f"sweep O b{b} h{hq}/{hkv} d{d} P{P} L{L} B{B}")
    err = np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse)
    assert np.all(err <= lse_bound(q, k)), "LSE beyond its bound"
    assert err.max() <= LSE_FIXED, f"LSE error {err.max()} beyond the fixed target"
    rb, kb, _ = M.mars_attn_tilelog_geometry(b, hq, hkv, d, P, L, B)
    exp = expected_tilelog_intervals(P, L, B, hq // hkv, rb, kb)
    log = log.cpu().numpy()
    for bi in range(b):
        for g in range(hkv):
            assert np.array_equal(log[bi, g], exp), (bi, g)


@pytest.mark.parametrize("b,hq,hkv,d,P,L,B,seed", BWD_SHAPES)
def test_sweep_backward(b, hq, hkv, d, P, L, B, seed):
    print(f"case sweep bwd b={b} hq={hq} hkv={hkv} d={d} P={P} L={L} B={B} seed={seed}", flush=True)
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, seed)
    do = I.small_grad_output(b, hq, d, P, L, seed)
    N = P + 2 * L
    qd, kd, vd, dod = q.to(dev()), k.to(dev()), v.to(dev()), do.to(dev())
    lse = torch.empty((b, hq, N), dtype=torch.float32, device=dev())
    od = M.mars_attn_fwd(qd, kd, vd, P, L, B, lse=lse)
    dq, dk, dv = M.mars_attn_bwd(qd, kd, vd, od, lse, dod, P, L, B)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = to_np64(q), to_np64(k), to_np64(v), to_np64(do)
    rq, rk, rv = O.attn_bwd(q64, k64, v64, do64, P, L, B)
    _, ref_lse = O.attn(q64, k64, v64, P, L, B)
    lse_err = np.minimum(lse_bound(q, k), np.abs(to_np64(lse) - ref_lse) + 1e-6)
    bq, bk, bv = bwd_bounds(q64, k64, v64, do64, to_np64(od), lse_err, P, L, B)
    for name, g, r, bb in (("dQ", dq, rq, bq), ("dK", dk, rk, bk), ("dV", dv, rv, bv)):
        check_bounded(to_np64(g), r, bb, f"sweep {name} b{b} h{hq}/{hkv} d{d} P{P} L{L} B{B}")


def _mid_bwd_shapes(n):
    """Backward layouts long enough that the dK/dV walks split into several chunks of tens of
    tiles (positions ~1000-4000), from a generator of their own so the cases above stay fixed."""
    rng = np.random.default_rng(20261203)
    out = []
    for _ in range(n):
        G = int(rng.choice([1, 2, 4, 7]))
        hkv = int(rng.integers(1, 3))
        d = int(rng.choice([64, 128]))
        P = int(rng.integers(0, 1500))
        L = int(rng.integers(200, 1200))
        B = int(rng.choice([1, 4, 8, 16, 32]))
        out.append((1, G * hkv, hkv, d, P, L, B, int(rng.integers(0, 1 << 30))))
    return out


MID_BWD_SHAPES = _mid_bwd_shapes(5)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("b,hq,hkv,d,P,L,B,seed", MID_BWD_SHAPES)
def test_sweep_backward_mid(b, hq, hkv, d, P, L, B, seed):
    """Whole dQ, dK, dV against the oracle at mid-size layouts (chunked walks, the
    longest-chunk-first grid)."""
    test_sweep_backward(b, hq, hkv, d, P, L, B, seed)


@pytest.mark.parametrize("batch,hq,hkv,d,W,cap,lens,seed", DEC_SHAPES)
def test_sweep_decode(batch, hq, hkv, d, W, cap, lens, seed):
    print(f"case sweep decode b={batch} hq={hq} hkv={hkv} d={d} W={W} cap={cap} lens={lens} seed={seed}", flush=True)
    s = I.DecodeShape("sweep", batch, hq, hkv, d, W, cap, 0, cap, 8, 0.95, 0.5, seed)
    x = I.decode_inputs(s, with_logits=False)
    cl = torch.tensor(lens, dtype=torch.int32)
    out = M.mars_decode_step(x.q_win.to(dev()), x.k_win.to(dev()), x.v_win.to(dev()), x.k_cache.to(dev()),
                             x.v_cache.to(dev()), cl.to(dev()))
    torch.cuda.synchronize()
    ref = O.decode(to_np64(x.q_win), to_np64(x.k_win), to_np64(x.v_win), to_np64(x.k_cache), to_np64(x.v_cache),
                   np.asarray(lens))
    check_close(to_np64(out), ref, f"sweep decode b{batch} h{hq}/{hkv} d{d} W{W} cap{cap}")


@pytest.mark.parametrize("batch,W,V,tau,seed", ACC_SHAPES)
def test_sweep_accept(batch, W, V, tau, seed):
    print(f"case sweep accept b={batch} W={W} V={V} tau={tau} seed={seed}", flush=True)
    lg = I.logits_inputs(batch, W, V, seed, spike_hi=12.0)
    Vp = -(-V // 8) * 8
    padded = torch.full((batch, W, Vp), -50.0, dtype=torch.bfloat16)
    padded[:, :, :V] = lg
    view = padded.to(dev())[:, :, :V]
    tok, pmax, n = M.mars_accept(view, tau)
    tok2, pmax2, mg, n2 = M.mars_accept_margin(view, tau)
    torch.cuda.synchronize()
    x64 = to_np64(lg)
    rtok, rpmax, rn = O.accept(x64, tau)
    _, _, rmg, rn2 = O.accept_margin(x64, tau)
    assert np.array_equal(tok.cpu().numpy(), rtok) and np.array_equal(tok2.cpu().numpy(), rtok)
    assert np.abs(pmax.cpu().numpy() - rpmax).max() <= PMAX_ABS
    assert np.abs(mg.cpu().numpy() - rmg).max() <= PMAX_ABS
    tie = tie_zone_sequences(rpmax, tau, tie_zone_width(pmax.cpu().numpy(), rpmax, tau))
    tie2 = tie_zone_sequences(np.where(rmg == 0.0, -np.inf, rmg), tau, tie_zone_width(mg.cpu().numpy(), rmg, tau))
    print(f"  tie-zone sequences: {int(tie.sum())} (pmax), {int(tie2.sum())} (margin)", flush=True)
    assert tie.sum() <= 1 and tie2.sum() <= 1
    assert np.array_equal(n.cpu().numpy()[~tie], rn[~tie])
    assert np.array_equal(n2.cpu().numpy()[~tie2], rn2[~tie2])
