"""GPU parity of mars_attn_fwd against the fp64 oracle.

Small shapes are compared on every output; the full-size workloads on sampled rows
(boundary positions plus random ones) in the launch configuration the bench times.
"""
import math

import numpy as np
import pytest
import torch

import structured_mask_attention_amd as M
from oracle import mars_oracle as O
from structured_mask_attention_amd import inputs as I
from tests.gpu_helpers import LSE_FIXED, check_close, dev, expected_tilelog, lse_bound, sample_rows, to_np64

pytestmark = pytest.mark.gpu


def run_case(b, hq, hkv, d, P, L, B, seed, dtype="bf16", rows=None, lse=True, want_inputs=False):
    print(f"case b={b} hq={hq} hkv={hkv} d={d} P={P} L={L} B={B} seed={seed} {dtype}", flush=True)
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, seed, dtype=dtype, in_scale=0.5 if dtype == "bf16" else 1.0)
    qd, kd, vd = q.to(dev()), k.to(dev()), v.to(dev())
    N = P + 2 * L
    lse_t = torch.empty((b, hq, N), dtype=torch.float32, device=dev()) if lse else None
    out = M.mars_attn_fwd(qd, kd, vd, P, L, B, lse=lse_t)
    torch.cuda.synchronize()
    ref, ref_lse = O.attn(to_np64(q), to_np64(k), to_np64(v), P, L, B, rows=rows)
    got = to_np64(out)
    got_lse = lse_t.cpu().numpy().astype(np.float64) if lse else None
    if rows is not None:
        got = got[:, rows]
        got_lse = got_lse[:, :, rows] if lse else None
    if want_inputs:
        return got, ref, got_lse, ref_lse, (q, k)
    return got, ref, got_lse, ref_lse


@pytest.mark.parametrize("b,hq,hkv,d,P,L,B", [
    (1, 1, 1, 64, 16, 64, 4),       # tiny layout in bf16
    (2, 7, 1, 64, 40, 150, 4),      # G = 7, ragged row tiles
    (1, 4, 4, 128, 0, 100, 8),      # no prompt, MHA
    (2, 8, 2, 128, 33, 70, 8),      # G = 4, L % B != 0... (70 % 8 = 6)
    (1, 2, 1, 64, 3, 37, 8),        # short last block
    (1, 3, 1, 128, 10, 5, 16),      # B > L
    (1, 2, 2, 64, 7, 33, 1),        # B = 1
    (1, 1, 1, 128, 0, 1, 1),        # N = 2
    (1, 2, 1, 64, 5, 0, 3),         # prompt only
    (1, 14, 2, 64, 64, 96, 4),      # Qwen2.5-0.5B heads, short
    (1, 28, 4, 128, 32, 160, 32),   # 7B heads, B = 32
])
def test_bf16_small_all_rows(b, hq, hkv, d, P, L, B):
    got, ref, got_lse, ref_lse, (q, k) = run_case(b, hq, hkv, d, P, L, B, seed=hash((b, hq, d, P, L, B)) % 1000,
                                                  want_inputs=True)
    check_close(got, ref, f"O b{b} h{hq}/{hkv} d{d} P{P} L{L} B{B}")
    err, bound = np.abs(got_lse - ref_lse), lse_bound(q, k)
    print(f"  lse max_abs={err.max():.3e} max_abs/bound={np.max(err / bound):.3f}", flush=True)
    assert np.all(err <= bound)
    assert err.max() <= LSE_FIXED


def test_fp32_tiny_workload():
    s = I.TINY
    q, k, v = I.train_inputs(s)
    out = M.mars_attn_fwd(q.to(dev()), k.to(dev()), v.to(dev()), s.P, s.L, s.B)
    torch.cuda.synchronize()
    ref, _ = O.attn(to_np64(q), to_np64(k), to_np64(v), s.P, s.L, s.B)
    mx, mean = check_close(to_np64(out), ref, "tiny fp32 [144,64]")
    assert mx <= 1e-4, "fp32 path should be far inside the bf16 bar"


@pytest.mark.parametrize("b,hq,hkv,d,P,L,B", [
    (2, 4, 2, 128, 40, 150, 8),     # head_dim 128, G = 2, ragged last workgroup
    (1, 3, 1, 128, 0, 100, 16),     # no prompt
    (1, 2, 2, 64, 300, 400, 32),    # long noisy stream: key tiles between the intervals skipped
    (2, 7, 1, 64, 70, 61, 5),       # G = 7, workgroups straddling P + L, short last block
    (1, 1, 1, 64, 5, 0, 3),         # prompt only
])
def test_fp32_layouts(b, hq, hkv, d, P, L, B):
    """The fp32 path (exact fp32, LDS key tiles over the union of a workgroup's two key
    intervals) on every row, O and LSE."""
    got, ref, got_lse, ref_lse = run_case(b, hq, hkv, d, P, L, B, seed=b * 1000 + P + L, dtype="fp32")
    mx, _ = check_close(got, ref, f"fp32 O b{b} h{hq}/{hkv} d{d} P{P} L{L} B{B}")
    assert mx <= 1e-4
    assert np.max(np.abs(got_lse - ref_lse)) <= 1e-4


@pytest.mark.parametrize("shape", [I.QWEN05B, I.QWEN7B, I.LONG7B], ids=lambda s: s.name)
def test_full_size_sampled_rows(shape):
    s = shape
    print(f"full size {s.name}", flush=True)
    q, k, v = I.train_inputs(s)
    qd, kd, vd = q.to(dev()), k.to(dev()), v.to(dev())
    out = M.mars_attn_fwd(qd, kd, vd, s.P, s.L, s.B)
    torch.cuda.synchronize()
    rows = sample_rows(s.P, s.L, s.B, n_random=48 if s.N > 8000 else 96, seed=s.seed)
    ref, _ = O.attn(to_np64(q), to_np64(k), to_np64(v), s.P, s.L, s.B, rows=rows)
    got = to_np64(out[:, torch.from_numpy(rows).to(dev())])
    check_close(got, ref, f"{s.name} sampled rows")
    # every output finite, and rows are convex combinations of V: |O| <= max |V|
    assert torch.isfinite(out.float()).all()
    assert float(out.float().abs().max()) <= float(v.float().abs().max()) * (1 + 2 ** -7)


@pytest.mark.parametrize("b,hq,hkv,d,P,L,B", [
    (1, 7, 1, 64, 40, 150, 4), (2, 8, 2, 128, 33, 70, 8), (1, 14, 2, 64, 256, 512, 4), (1, 3, 1, 128, 10, 5, 16),
    (1, 2, 2, 64, 0, 64, 32)])
def test_tile_log_matches_oracle(b, hq, hkv, d, P, L, B):
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, seed=7)
    _, log = M.mars_attn_fwd_tilelog(q.to(dev()), k.to(dev()), v.to(dev()), P, L, B)
    torch.cuda.synchronize()
    rb, kb, _ = M.mars_attn_tilelog_geometry(b, hq, hkv, d, P, L, B)
    exp = expected_tilelog(P, L, B, hq // hkv, rb, kb)
    log = log.cpu().numpy()
    for bi in range(b):
        for g in range(hkv):
            assert np.array_equal(log[bi, g], exp), (bi, g)


def test_strided_views_and_canaries():
    """q/k/v as views of one packed [b, N, Hq+2Hkv, D] buffer; output inside guard bytes."""
    b, hq, hkv, d, P, L, B = 2, 8, 2, 128, 20, 60, 4
    N = P + 2 * L
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, seed=11)
    packed = torch.cat([q, k, v], dim=2).to(dev())
    qv, kv, vv = packed[:, :, :hq], packed[:, :, hq:hq + hkv], packed[:, :, hq + hkv:]
    guard = 4096
    buf = torch.full((guard + b * N * hq * d + guard,), 12345, dtype=torch.int16, device=dev())
    out = buf[guard:guard + b * N * hq * d].view(torch.bfloat16).view(b, N, hq, d)
    M.mars_attn_fwd(qv, kv, vv, P, L, B, out=out)
    torch.cuda.synchronize()
    assert (buf[:guard] == 12345).all() and (buf[-guard:] == 12345).all()
    ref, _ = O.attn(to_np64(q), to_np64(k), to_np64(v), P, L, B)
    check_close(to_np64(out), ref, "strided")


def test_deterministic():
    s = I.QWEN05B
    q, k, v = (t.to(dev()) for t in I.train_inputs(s))
    o1 = M.mars_attn_fwd(q, k, v, s.P, s.L, s.B)
    o2 = M.mars_attn_fwd(q, k, v, s.P, s.L, s.B)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_noisy_blocks_match_decode_step():
    """Noisy block k of the training layout == decode step on cache [0, P+kB) + window block k."""
    b, hq, hkv, d, P, L, B = 2, 7, 1, 128, 24, 40, 4
    N = P + 2 * L
    q, k, v = (t.to(dev()) for t in I.small_train_inputs(b, hq, hkv, d, P, L, seed=5))
    o_train = M.mars_attn_fwd(q, k, v, P, L, B)
    cap = P + L
    kc = k[:, :cap].permute(0, 2, 1, 3).contiguous()
    vc = v[:, :cap].permute(0, 2, 1, 3).contiguous()
    for blk in range(L // B):
        r0 = P + L + blk * B
        lens = torch.full((b,), P + blk * B, dtype=torch.int32, device=dev())
        o_dec = M.mars_decode_step(q[:, r0:r0 + B].contiguous(), k[:, r0:r0 + B].contiguous(),
                                   v[:, r0:r0 + B].contiguous(), kc, vc, lens)
        torch.cuda.synchronize()
        diff = (o_dec.float() - o_train[:, r0:r0 + B].float()).abs()
        assert float(diff.max()) <= 2e-2 and float(diff.mean()) <= 2e-3, blk


def test_empty_inputs_are_noops():
    q = torch.zeros((0, 10, 2, 64), dtype=torch.bfloat16, device=dev())
    M.mars_attn_fwd(q, q[:, :, :1], q[:, :, :1], 2, 4, 2)
    q2 = torch.zeros((1, 0, 2, 64), dtype=torch.bfloat16, device=dev())
    M.mars_attn_fwd(q2, q2[:, :, :1], q2[:, :, :1], 0, 0, 2)
    torch.cuda.synchronize()


@pytest.mark.parametrize("d,low", [(64, 1000.0), (128, 1000.0), (64, 200.0), (128, 200.0)])
def test_bf16_running_max_moves_late(d, low):
    """Keys 0..31 (the first key tile of every row) score far below all later keys: every
    q has component 0 equal to 1 and those keys have component 0 equal to -low.  A row's
    running max then comes from tile 0 and the later tiles' P exceed it by up to ~2^180
    (low = 1000: the kernel must move the max in a later tile) or ~2^40 (low = 200: P > 1
    without a rescale).  The dominant scores stay moderate, so the single bf16 rounding of
    Q*scale keeps its usual small effect; checked against the fp64 oracle on every output."""
    b, hq, hkv, P, L, B = 1, 7, 1, 24, 72, 4
    print(f"case running max d={d} low={low}", flush=True)
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, seed=777 + d, dtype="bf16", in_scale=0.5)
    N = P + 2 * L
    qf, kf = q.float(), k.float()
    qf[..., 0] = 1.0
    kf[..., 0] = 0.0
    kf[:, :32, :, 0] = -low
    q, k = qf.to(torch.bfloat16), kf.to(torch.bfloat16)
    lse_t = torch.empty((b, hq, N), dtype=torch.float32, device=dev())
    out = M.mars_attn_fwd(q.to(dev()), k.to(dev()), v.to(dev()), P, L, B, lse=lse_t)
    torch.cuda.synchronize()
    ref, ref_lse = O.attn(to_np64(q), to_np64(k), to_np64(v), P, L, B)
    check_close(to_np64(out), ref, f"O running max d{d} low{low}")
    err = np.abs(lse_t.cpu().numpy().astype(np.float64) - ref_lse)
    bound = lse_bound(q, k)
    print(f"  lse max_abs={err.max():.3e} max_abs/bound={np.max(err / bound):.3f}", flush=True)
    assert np.all(err <= bound)


@pytest.mark.parametrize("d,high,where", [(64, 600.0, "late"), (128, 600.0, "late"), (64, 600.0, "all"),
                                          (128, 600.0, "all"), (64, -600.0, "all")])
def test_bf16_large_scores(d, high, where):
    """Scores far from 0 in the log2 domain: every q has component 0 equal to 1 and keys get
    component 0 equal to `high` (scale*log2(e)*600 ~ 108).  "late": only keys 64..95, so rows
    start with moderate scores and a later tile's P sum passes 2^64 (the row's offset must
    move there); "all": every key, so rows start with a first max beyond +-64 (large
    positive, or large negative for high < 0) and carry a nonzero offset from their first
    tile.  Checked against the fp64 oracle on every output and on the LSE."""
    b, hq, hkv, P, L, B = 1, 7, 1, 24, 72, 4
    print(f"case large scores d={d} high={high} {where}", flush=True)
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, seed=991 + d, dtype="bf16", in_scale=0.5)
    N = P + 2 * L
    qf, kf = q.float(), k.float()
    qf[..., 0] = 1.0
    kf[..., 0] = 0.0
    if where == "late":
        kf[:, 64:96, :, 0] = high
    else:
        kf[..., 0] = high
    q, k = qf.to(torch.bfloat16), kf.to(torch.bfloat16)
    lse_t = torch.empty((b, hq, N), dtype=torch.float32, device=dev())
    out = M.mars_attn_fwd(q.to(dev()), k.to(dev()), v.to(dev()), P, L, B, lse=lse_t)
    torch.cuda.synchronize()
    ref, ref_lse = O.attn(to_np64(q), to_np64(k), to_np64(v), P, L, B)
    check_close(to_np64(out), ref, f"O large scores d{d} high{high} {where}")
    err = np.abs(lse_t.cpu().numpy().astype(np.float64) - ref_lse)
    bound = lse_bound(q, k)
    print(f"  lse max_abs={err.max():.3e} max_abs/bound={np.max(err / bound):.3f}", flush=True)
    assert np.all(err <= bound)
