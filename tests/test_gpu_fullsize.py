"""Whole-output GPU parity at the full training-layout sizes, in the launch configuration the
bench times (MARS §3.2 Eq. 2: the mask whose tiles the kernel skips).

* every element of O and LSE of the Qwen2.5-0.5B- and 7B-shaped layouts;
* every row of two whole KV groups (14 of the 28 query heads) of the long layout;
* the kernel's visited-tile log, bit for bit, on the three layouts and on one layout whose
  rows see more than 32768 keys (more than 1024 key tiles per walk);
* every dQ row and every dK/dV key of one (batch, KV group) of the 0.5B and the 7B layouts'
  backward.

The oracle runs one (batch, head) slice per thread (tests/gpu_helpers.py).
"""
import numpy as np
import pytest
import torch

import structured_mask_attention_amd as M
from oracle import mars_oracle as O
from structured_mask_attention_amd import inputs as I
from tests.gpu_helpers import (LSE_FIXED, bwd_bounds, check_bounded, check_close, dev, expected_tilelog_intervals,
                               lse_bound, lse_bound_slices, oracle_attn_slices, to_np64)

pytestmark = pytest.mark.gpu


def _whole(s, pairs):
    print(f"case whole output {s.name}: {len(pairs)} (batch, head) slices", flush=True)
    q, k, v = I.train_inputs(s)
    lse = torch.empty((s.batch, s.hq, s.N), dtype=torch.float32, device=dev())
    out = M.mars_attn_fwd(q.to(dev()), k.to(dev()), v.to(dev()), s.P, s.L, s.B, lse=lse)
    torch.cuda.synchronize()
    got, got_lse = to_np64(out), lse.cpu().numpy().astype(np.float64)
    del out, lse
    q64, k64, v64 = to_np64(q), to_np64(k), to_np64(v)
    ref = oracle_attn_slices(q64, k64, v64, s.P, s.L, s.B, pairs)
    bnd = lse_bound_slices(q64, k64, pairs)
    go = np.stack([got[b, :, h] for b, h in pairs])
    ro = np.stack([ref[(b, h)][0] for b, h in pairs])
    check_close(go, ro, f"{s.name} O, {len(pairs)} whole slices")
    worst = worst_abs = 0.0
    for b, h in pairs:
        err = np.abs(got_lse[b, h] - ref[(b, h)][1])
        ratio = float(np.max(err / bnd[(b, h)]))
        worst = max(worst, ratio)
        worst_abs = max(worst_abs, float(err.max()))
        assert ratio <= 1.0, f"LSE b{b} h{h}: error/bound {ratio:.3f}"
    print(f"  lse max err/bound={worst:.3f} max abs={worst_abs:.3e} nats", flush=True)
    assert worst_abs <= LSE_FIXED


@pytest.mark.timeout(600)
@pytest.mark.parametrize("shape", [I.QWEN05B, I.QWEN7B], ids=lambda s: s.name)
def test_whole_output(shape):
    """Every O and LSE element of the layout (all batches, all heads, all positions)."""
    s = shape
    _whole(s, [(b, h) for b in range(s.batch) for h in range(s.hq)])


@pytest.mark.timeout(600)
def test_long_layout_whole_kv_groups():
    """Every row of KV groups 0 and 3 of the long layout (query heads 0-6 and 21-27)."""
    s = I.LONG7B
    G = s.hq // s.hkv
    _whole(s, [(0, h) for h in list(range(G)) + list(range(3 * G, 4 * G))])


def _tilelog_case(b, hq, hkv, d, P, L, B, seed, rows_check=None):
    N = P + 2 * L
    print(f"case tile log b={b} hq={hq} hkv={hkv} d={d} P={P} L={L} B={B} N={N}", flush=True)
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, seed)
    qd, kd, vd = q.to(dev()), k.to(dev()), v.to(dev())
    o_log, log = M.mars_attn_fwd_tilelog(qd, kd, vd, P, L, B)
    o_plain = M.mars_attn_fwd(qd, kd, vd, P, L, B)
    torch.cuda.synchronize()
    rb, kb, _ = M.mars_attn_tilelog_geometry(b, hq, hkv, d, P, L, B)
    exp = expected_tilelog_intervals(P, L, B, hq // hkv, rb, kb)
    log = log.cpu().numpy()
    for bi in range(b):
        for g in range(hkv):
            bad = np.argwhere(log[bi, g] != exp)
            assert bad.size == 0, f"tile log b{bi} g{g}: {len(bad)} tiles differ, first {bad[:4].tolist()}"
    # the logging instantiation computes the same output as the plain one, bit for bit
    assert torch.equal(o_log.view(torch.int16), o_plain.view(torch.int16))
    n_vis = int((log > 0).sum())
    print(f"  {log.size} tiles, {n_vis} visited, {int((log == 2).sum())} unmasked", flush=True)
    if rows_check is not None:
        ref, _ = O.attn(to_np64(q), to_np64(k), to_np64(v), P, L, B, rows=rows_check)
        check_close(to_np64(o_plain[:, torch.from_numpy(rows_check).to(dev())]), ref, "sampled rows")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("shape", [I.QWEN05B, I.QWEN7B, I.LONG7B], ids=lambda s: s.name)
def test_tilelog_full_size(shape):
    """Bit-exact visited-tile log at the full layout (batch 8 at 0.5B, where the grid exceeds
    the resident slots; 112 and 480 key tiles at 7B and the long layout, so the per-lane class
    lookup for key tiles 64 and beyond is taken)."""
    s = shape
    _tilelog_case(s.batch, s.hq, s.hkv, s.d, s.P, s.L, s.B, s.seed)


@pytest.mark.timeout(300)
def test_tilelog_beyond_1024_key_tiles():
    """Rows that see more than 32768 keys: a walk longer than 1024 key tiles, whose tiles past
    the 1024th are classified on the spot instead of from the per-lane table."""
    P, L, B = 32800, 64, 8
    N = P + 2 * L
    rows = np.array([0, 31, 32767, 32768, P - 1, P, P + L - 1, P + L, P + L + B - 1, N - 2, N - 1])
    _tilelog_case(1, 2, 1, 64, P, L, B, seed=4242, rows_check=rows)


def _bwd_whole_pair(s, bsel, g):
    G = s.hq // s.hkv
    hs = slice(g * G, (g + 1) * G)
    print(f"case bwd whole pair {s.name} b={bsel} g={g}", flush=True)
    q, k, v = I.train_inputs(s)
    do = I.grad_output(s)
    qd, kd, vd, dod = q.to(dev()), k.to(dev()), v.to(dev()), do.to(dev())
    lse = torch.empty((s.batch, s.hq, s.N), dtype=torch.float32, device=dev())
    od = M.mars_attn_fwd(qd, kd, vd, s.P, s.L, s.B, lse=lse)
    dq, dk, dv = M.mars_attn_bwd(qd, kd, vd, od, lse, dod, s.P, s.L, s.B)
    torch.cuda.synchronize()
    q64 = to_np64(q[bsel:bsel + 1, :, hs])
    k64 = to_np64(k[bsel:bsel + 1, :, g:g + 1])
    v64 = to_np64(v[bsel:bsel + 1, :, g:g + 1])
    do64 = to_np64(do[bsel:bsel + 1, :, hs])
    rq, rk, rv = O.attn_bwd(q64, k64, v64, do64, s.P, s.L, s.B)
    o64 = to_np64(od[bsel:bsel + 1, :, hs])
    lse_err = lse_bound(q[bsel:bsel + 1, :, hs], k[bsel:bsel + 1, :, g:g + 1])
    bq, bk, bv = bwd_bounds(q64, k64, v64, do64, o64, lse_err, s.P, s.L, s.B)
    for name, got, ref, bnd in (("dq", dq[bsel:bsel + 1, :, hs], rq, bq), ("dk", dk[bsel:bsel + 1, :, g:g + 1], rk, bk),
                                ("dv", dv[bsel:bsel + 1, :, g:g + 1], rv, bv)):
        check_bounded(to_np64(got), ref, bnd, f"{s.name} {name} b{bsel} g{g} whole")
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()


@pytest.mark.timeout(600)
def test_bwd_whole_pair_qwen05b():
    """Every dQ row (7 heads) and every dK/dV key of batch 7, KV group 1 of the 0.5B layout's
    backward, from one launch over the whole workload."""
    _bwd_whole_pair(I.QWEN05B, 7, 1)


@pytest.mark.timeout(600)
def test_bwd_whole_pair_qwen7b():
    """Every dQ row (7 heads) and every dK/dV key of batch 1, KV group 2 of the 7B layout's
    backward (head_dim 128: 192-key blocks, walks split into chunks whose partials are
    summed by the last arrival), from one launch over the whole workload."""
    _bwd_whole_pair(I.QWEN7B, 1, 2)
