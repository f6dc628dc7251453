"""GPU parity of mars_attn_bwd against the fp64 oracle's gradients.

Small shapes are compared on every element; the full-size workloads on sampled query rows
(dQ) and sampled keys (dK, dV) in the launch configuration the bench times.  Each element
must lie within a bound derived from the kernel's roundings (tests/gpu_helpers.bwd_bounds).
The kernel takes O and the LSE as inputs: "isolated" cases hand it the oracle's O (rounded
to bf16) and LSE (fp32), "end to end" cases the forward kernel's own outputs.
"""
import numpy as np
import pytest
import torch

import structured_mask_attention_amd as M
from oracle import mars_oracle as O
from structured_mask_attention_amd import inputs as I
from tests.gpu_helpers import bwd_bounds, check_bounded, dev, lse_bound, to_np64

pytestmark = pytest.mark.gpu


def run_bwd(q, k, v, do, P, L, B, source, rows=None, keys=None):
    """Backward on the GPU; returns the kernel's gradients (float64, restricted to rows /
    keys), the oracle's, and the error bounds."""
    qd, kd, vd, dod = q.to(dev()), k.to(dev()), v.to(dev()), do.to(dev())
    b, N, hq, d = q.shape
    q64, k64, v64, do64 = to_np64(q), to_np64(k), to_np64(v), to_np64(do)
    ref_o, ref_lse = O.attn(q64, k64, v64, P, L, B)
    if source == "oracle":
        od = torch.from_numpy(ref_o).to(torch.bfloat16).to(dev())
        lsed = torch.from_numpy(ref_lse).to(torch.float32).to(dev())
        lse_err = np.abs(to_np64(lsed) - ref_lse) + 1e-6
    else:
        lsed = torch.empty((b, hq, N), dtype=torch.float32, device=dev())
        od = M.mars_attn_fwd(qd, kd, vd, P, L, B, lse=lsed)
        torch.cuda.synchronize()
        lse_err = np.minimum(lse_bound(q, k), np.abs(to_np64(lsed) - ref_lse) + 1e-6)
    dq, dk, dv = M.mars_attn_bwd(qd, kd, vd, od, lsed, dod, P, L, B)
    torch.cuda.synchronize()
    gq, gk, gv = to_np64(dq), to_np64(dk), to_np64(dv)
    if rows is not None:
        gq = gq[:, rows]
    if keys is not None:
        gk, gv = gk[:, keys], gv[:, keys]
    rq, rk, rv = O.attn_bwd(q64, k64, v64, do64, P, L, B, rows=rows, keys=keys)
    bq, bk, bv = bwd_bounds(q64, k64, v64, do64, to_np64(od), lse_err, P, L, B, rows=rows, keys=keys)
    return (gq, gk, gv), (rq, rk, rv), (bq, bk, bv)


def check_all(got, ref, bnd, tag):
    for name, g, r, bb in zip(("dQ", "dK", "dV"), got, ref, bnd):
        check_bounded(g, r, bb, f"{name} {tag}")


@pytest.mark.parametrize("b,hq,hkv,d,P,L,B", [
    (1, 1, 1, 64, 16, 64, 4),       # tiny layout in bf16
    (2, 7, 1, 64, 40, 150, 4),      # G = 7, ragged position and key tiles
    (1, 4, 4, 128, 0, 100, 8),      # no prompt, MHA
    (2, 8, 2, 128, 33, 70, 8),      # G = 4, short last block
    (1, 2, 1, 64, 3, 37, 8),        # short last block
    (1, 3, 1, 128, 10, 5, 16),      # B > L
    (1, 2, 2, 64, 7, 33, 1),        # B = 1
    (1, 1, 1, 128, 0, 1, 1),        # N = 2
    (1, 2, 1, 64, 5, 0, 3),         # prompt only
    (1, 14, 2, 64, 64, 96, 4),      # Qwen2.5-0.5B heads, short
    (1, 28, 4, 128, 32, 160, 32),   # 7B heads, B = 32
    (1, 2, 1, 64, 130, 120, 4),     # key blocks straddling P and P + L
])
def test_bwd_small_all_elements(b, hq, hkv, d, P, L, B):
    seed = hash((b, hq, d, P, L, B)) % 1000
    print(f"case bwd b={b} hq={hq} hkv={hkv} d={d} P={P} L={L} B={B} seed={seed}", flush=True)
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, seed)
    do = I.small_grad_output(b, hq, d, P, L, seed)
    got, ref, bnd = run_bwd(q, k, v, do, P, L, B, "oracle")
    check_all(got, ref, bnd, f"b{b} h{hq}/{hkv} d{d} P{P} L{L} B{B}")


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_end_to_end_with_forward_outputs(d):
    """O and LSE from mars_attn_fwd itself (the training use)."""
    b, hq, hkv, P, L, B = 2, 14, 2, 48, 80, 4
    print(f"case bwd end to end d={d}", flush=True)
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, 4242 + d)
    do = I.small_grad_output(b, hq, d, P, L, 4242 + d)
    got, ref, bnd = run_bwd(q, k, v, do, P, L, B, "forward")
    check_all(got, ref, bnd, f"end-to-end d{d}")


def test_bwd_closed_form_constant_v():
    """Every key carries the same V: dQ = dK = 0 exactly in exact arithmetic, so the kernel's
    dQ and dK are pure rounding noise, far below the gradients' usual scale."""
    b, hq, hkv, d, P, L, B = 1, 7, 1, 64, 24, 72, 4
    print("case bwd constant V", flush=True)
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, 77)
    v = v[:, :1].expand_as(v).contiguous()
    do = I.small_grad_output(b, hq, d, P, L, 77)
    got, ref, bnd = run_bwd(q, k, v, do, P, L, B, "oracle")
    check_all(got, ref, bnd, "constant V")
    assert np.max(np.abs(ref[0])) < 1e-12 and np.max(np.abs(ref[1])) < 1e-12


def test_bwd_deterministic():
    b, hq, hkv, d, P, L, B = 2, 14, 2, 64, 32, 64, 4
    q, k, v = (t.to(dev()) for t in I.small_train_inputs(b, hq, hkv, d, P, L, 5))
    do = I.small_grad_output(b, hq, d, P, L, 5).to(dev())
    lse = torch.empty((b, hq, P + 2 * L), dtype=torch.float32, device=dev())
    o = M.mars_attn_fwd(q, k, v, P, L, B, lse=lse)
    a = M.mars_attn_bwd(q, k, v, o, lse, do, P, L, B)
    c = M.mars_attn_bwd(q, k, v, o, lse, do, P, L, B)
    torch.cuda.synchronize()
    for x, y in zip(a, c):
        assert torch.equal(x, y)


@pytest.mark.parametrize("shape", [I.QWEN05B, I.QWEN7B, I.LONG7B], ids=lambda s: s.name)
def test_bwd_deterministic_full_size(shape):
    """The full-size layouts, whose heavy key blocks are walked in several chunks reduced by
    the last-arriving wave: three launches (the second into a workspace filled with garbage
    first) give bit-identical dQ, dK and dV, whatever order the chunks finish in."""
    s = shape
    print(f"case bwd deterministic {s.name}", flush=True)
    plan = M.mars_attn_bwd_plan(s.batch, s.hq, s.hkv, s.d, s.P, s.L, s.B)
    assert plan["max_chunks"] > 1
    q, k, v = (t.to(dev()) for t in I.train_inputs(s))
    do = I.grad_output(s).to(dev())
    lse = torch.empty((s.batch, s.hq, s.N), dtype=torch.float32, device=dev())
    o = M.mars_attn_fwd(q, k, v, s.P, s.L, s.B, lse=lse)
    ws = torch.empty(M.mars_attn_bwd_workspace_bytes(s.batch, s.hq, s.hkv, s.d, s.P, s.L, s.B), dtype=torch.uint8,
                     device=dev())
    first = [t.clone() for t in M.mars_attn_bwd(q, k, v, o, lse, do, s.P, s.L, s.B, ws=ws)]
    for fill in (0xA5, None):
        if fill is not None:
            ws.fill_(fill)
        again = M.mars_attn_bwd(q, k, v, o, lse, do, s.P, s.L, s.B, ws=ws)
        torch.cuda.synchronize()
        for x, y in zip(first, again):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16))


def _head_major(x):
    """x [b, N, H, D] copied into head-major storage with one spare head: a [b, N, H, D] view
    whose position stride is D and head stride N * D."""
    bb, n, h, d = x.shape
    big = torch.zeros((bb, h + 1, n, d), dtype=x.dtype, device=x.device)
    big[:, :h] = x.permute(0, 2, 1, 3)
    return big[:, :h].permute(0, 2, 1, 3)


def test_bwd_strided_views():
    """Gradient outputs and dO as strided views of larger buffers (head-major storage);
    the padding around them stays untouched."""
    b, hq, hkv, d, P, L, B = 1, 4, 2, 64, 8, 40, 4
    N = P + 2 * L
    q, k, v = (t.to(dev()) for t in I.small_train_inputs(b, hq, hkv, d, P, L, 9))
    do_c = I.small_grad_output(b, hq, d, P, L, 9).to(dev())
    lse = torch.empty((b, hq, N), dtype=torch.float32, device=dev())
    o = M.mars_attn_fwd(q, k, v, P, L, B, lse=lse)
    ref = M.mars_attn_bwd(q, k, v, o, lse, do_c, P, L, B)
    do_v = _head_major(do_c)
    bufs = [torch.full((b, h + 1, N, d), 7.0, dtype=torch.bfloat16, device=dev()) for h in (hq, hkv, hkv)]
    views = [buf[:, :h].permute(0, 2, 1, 3) for buf, h in zip(bufs, (hq, hkv, hkv))]
    M.mars_attn_bwd(q, k, v, o, lse, do_v, P, L, B, dq=views[0], dk=views[1], dv=views[2])
    torch.cuda.synchronize()
    for r, vw, buf, h in zip(ref, views, bufs, (hq, hkv, hkv)):
        assert torch.equal(r, vw)
        assert torch.all(buf[:, h:] == 7.0)


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_strided_inputs(d):
    """Q, K, V, O and dO all head-major views (position stride D, head stride N*D): the
    dK/dV kernels copy the caller's Q and dO tiles with those strides, rows past N (N = 88,
    a ragged last tile) repeating row N - 1.  Bit-identical to the contiguous call."""
    b, hq, hkv, P, L, B = 2, 4, 2, 8, 40, 4
    N = P + 2 * L
    print(f"case bwd strided inputs d={d} N={N}", flush=True)
    q, k, v = (t.to(dev()) for t in I.small_train_inputs(b, hq, hkv, d, P, L, 19))
    do_c = I.small_grad_output(b, hq, d, P, L, 19).to(dev())
    lse = torch.empty((b, hq, N), dtype=torch.float32, device=dev())
    o = M.mars_attn_fwd(q, k, v, P, L, B, lse=lse)
    ref = M.mars_attn_bwd(q, k, v, o, lse, do_c, P, L, B)
    qs, ks, vs, os_, dos = (_head_major(t) for t in (q, k, v, o, do_c))
    assert qs.stride(1) == d and qs.stride(2) == N * d
    got = M.mars_attn_bwd(qs, ks, vs, os_, lse, dos, P, L, B)
    torch.cuda.synchronize()
    for r, g_ in zip(ref, got):
        assert torch.equal(r, g_)


@pytest.mark.timeout(300)
@pytest.mark.parametrize("P,kblk", [(16384, 110), (26000, 180)], ids=["list804", "closed1064"])
def test_bwd_long_walk_order(P, kblk):
    """Head_dim 64, one KV head, long prompts.  N = 16512: 129 key blocks x 8 chunks exceed the
    launch's 1024-entry work list, but only 804 (key block, chunk) entries exist, so the list is
    used.  N = 26128: 205 key blocks, 1064 entries, so dK/dV take the closed-form grid order.
    dQ on sampled rows; dK/dV on keys whose rows the oracle affords: key block kblk, whose walk
    is split into chunks, the end of the prompt and the noisy stream.  Over every key of the KV
    head, at any size: sum_j dV_j = sum_i dO_i (rows of P sum to one) and sum_j dK_j = 0 (rows
    of dS sum to zero).  Two launches bit-identical."""
    b, hq, hkv, d, L, B = 1, 2, 1, 64, 64, 8
    N = P + 2 * L
    assert M.mars_attn_bwd_plan(b, hq, hkv, d, P, L, B)["work_list"] == (P == 16384)
    print(f"case bwd long walk order d={d} P={P} L={L} B={B} N={N}", flush=True)
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, 77)
    do = I.small_grad_output(b, hq, d, P, L, 77)
    qd, kd, vd, dod = q.to(dev()), k.to(dev()), v.to(dev()), do.to(dev())
    lse = torch.empty((b, hq, N), dtype=torch.float32, device=dev())
    od = M.mars_attn_fwd(qd, kd, vd, P, L, B, lse=lse)
    dq, dk, dv = M.mars_attn_bwd(qd, kd, vd, od, lse, dod, P, L, B)
    again = M.mars_attn_bwd(qd, kd, vd, od, lse, dod, P, L, B)
    torch.cuda.synchronize()
    for x, y in zip((dq, dk, dv), again):
        assert torch.equal(x, y)
    from tests.gpu_helpers import sample_rows
    rows = sample_rows(P, L, B, 12, 77)
    keys = np.array([kblk * 128, kblk * 128 + 1, kblk * 128 + 63, (kblk + 1) * 128 - 1, P - 1, P, P + L - 1, P + L, N - 1])
    q64, k64, v64, do64 = (to_np64(t) for t in (q, k, v, do))
    rq, rk, rv = O.attn_bwd(q64, k64, v64, do64, P, L, B, rows=rows, keys=keys)
    bq, bk, bv = bwd_bounds(q64, k64, v64, do64, to_np64(od), lse_bound(q, k), P, L, B, rows=rows, keys=keys)
    check_all((to_np64(dq)[:, rows], to_np64(dk)[:, keys], to_np64(dv)[:, keys]), (rq, rk, rv), (bq, bk, bv),
              "long walk order")
    # identities over all keys (per KV head; bf16 outputs: tolerance 2^-7 of the magnitude sums)
    gdv, gdk = to_np64(dv)[0, :, 0], to_np64(dk)[0, :, 0]
    sdo = do64[0].sum(axis=(0, 1))
    assert np.all(np.abs(gdv.sum(axis=0) - sdo) <= 2.0 ** -7 * (np.abs(gdv).sum(axis=0) + np.abs(do64[0]).sum(axis=(0, 1))))
    assert np.all(np.abs(gdk.sum(axis=0)) <= 2.0 ** -7 * np.abs(gdk).sum(axis=0))


@pytest.mark.parametrize("shape", [I.QWEN05B, I.QWEN7B, I.LONG7B], ids=lambda s: s.name)
def test_bwd_full_size_sampled(shape):
    """Full-size workloads, batch element 0 and KV group 0 (the others are independent and
    computed by the same launch): dQ on boundary and random positions of every head of the
    group; dK/dV on keys whose rows the oracle can afford (all of them for 0.5B; for the
    long layout keys of the noisy stream and the end of the clean one)."""
    s = shape
    print(f"case bwd full size {s.name}", flush=True)
    q, k, v = I.train_inputs(s)
    do = I.grad_output(s)
    G = s.hq // s.hkv
    P, L, B, N = s.P, s.L, s.B, s.N
    rng = np.random.default_rng(s.seed)
    from tests.gpu_helpers import sample_rows
    rows = sample_rows(P, L, B, 12, s.seed)
    if N <= 4096:
        keys = np.unique(np.concatenate([[0, P - 1, P, P + L - 1, P + L, N - 1], rng.integers(0, N, 10)]))
    else:
        keys = np.unique(np.concatenate([[P + L - 1, P + L, N - B, N - 1], rng.integers(P + L, N, 8)]))
    # Run the whole workload on the GPU; compare batch 0, KV group 0.
    qd, kd, vd, dod = q.to(dev()), k.to(dev()), v.to(dev()), do.to(dev())
    lsed = torch.empty((s.batch, s.hq, N), dtype=torch.float32, device=dev())
    od = M.mars_attn_fwd(qd, kd, vd, P, L, B, lse=lsed)
    dq, dk, dv = M.mars_attn_bwd(qd, kd, vd, od, lsed, dod, P, L, B)
    torch.cuda.synchronize()
    sl = slice(0, G)
    q64, k64, v64, do64 = (to_np64(t[:1, :, sl] if t.shape[2] == s.hq else t[:1, :, :1]) for t in (q, k, v, do))
    gq = to_np64(dq[:1, :, sl])[:, rows]
    gk, gv = to_np64(dk[:1, :, :1])[:, keys], to_np64(dv[:1, :, :1])[:, keys]
    rq, rk, rv = O.attn_bwd(q64, k64, v64, do64, P, L, B, rows=rows, keys=keys)
    o64 = to_np64(od[:1, :, sl])
    lse_err = lse_bound(q[:1, :, sl], k[:1, :, :1])
    bq, bk, bv = bwd_bounds(q64, k64, v64, do64, o64, lse_err, P, L, B, rows=rows, keys=keys)
    check_all((gq, gk, gv), (rq, rk, rv), (bq, bk, bv), s.name)
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all()
