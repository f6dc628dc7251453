"""Softmax scales other than the default 1/sqrt(head_dim), through every attention entry point,
against the fp64 oracle at the same scale: the training forward (bf16 and fp32, O and LSE),
its backward, and the decode step (with and without a workspace).  The scale multiplies the
scores of Eq. 2's masked softmax before the exponential, so a kernel that kept the default,
or applied the given value to only some of its products (the scores, dQ, dK, the decode
chunks or the window keys), fails these cases while every default-scale test still passes.
"""
import numpy as np
import pytest
import torch

import structured_mask_attention_amd as M
from oracle import mars_oracle as O
from structured_mask_attention_amd import inputs as I
from tests.gpu_helpers import LSE_FIXED, bwd_bounds, check_bounded, check_close, dev, lse_bound, to_np64

pytestmark = pytest.mark.gpu

# Against the defaults 0.125 (head_dim 64) and 0.088 (head_dim 128): well below and well above.
SCALES = [0.03, 0.3]


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("d", [64, 128])
def test_forward_scale_bf16(d, scale):
    b, hq, hkv, P, L, B = 2, 8, 2, 24, 70, 8
    N = P + 2 * L
    print(f"case fwd scale={scale} d={d}", flush=True)
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, 31 + d, dtype="bf16", in_scale=0.5)
    lse = torch.empty((b, hq, N), dtype=torch.float32, device=dev())
    out = M.mars_attn_fwd(q.to(dev()), k.to(dev()), v.to(dev()), P, L, B, scale=scale, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = O.attn(to_np64(q), to_np64(k), to_np64(v), P, L, B, scale=scale)
    check_close(to_np64(out), ref, f"O scale {scale} d{d}")
    err, bound = np.abs(to_np64(lse) - ref_lse), lse_bound(q, k, scale=scale)
    print(f"  lse max_abs={err.max():.3e} max_abs/bound={np.max(err / bound):.3f}", flush=True)
    assert np.all(err <= bound)
    assert err.max() <= LSE_FIXED
    # the default-scale result differs by far more than the tolerance: the scale is applied
    dflt = M.mars_attn_fwd(q.to(dev()), k.to(dev()), v.to(dev()), P, L, B)
    torch.cuda.synchronize()
    assert np.abs(to_np64(dflt) - ref).max() > 0.1


@pytest.mark.parametrize("scale", SCALES)
def test_forward_scale_fp32(scale):
    b, hq, hkv, d, P, L, B = 1, 4, 2, 64, 40, 52, 4
    N = P + 2 * L
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, 57, dtype="fp32", in_scale=1.0)
    lse = torch.empty((b, hq, N), dtype=torch.float32, device=dev())
    out = M.mars_attn_fwd(q.to(dev()), k.to(dev()), v.to(dev()), P, L, B, scale=scale, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = O.attn(to_np64(q), to_np64(k), to_np64(v), P, L, B, scale=scale)
    mx, _ = check_close(to_np64(out), ref, f"fp32 O scale {scale}")
    assert mx <= 1e-4
    assert np.max(np.abs(to_np64(lse) - ref_lse)) <= 1e-4


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("d", [64, 128])
def test_backward_scale(d, scale):
    """dQ = scale dS K and dK = scale dS^T Q on top of P at the given scale; O and LSE from the
    oracle at that scale, every element within the kernel's rounding bounds."""
    b, hq, hkv, P, L, B = 1, 4, 2, 16, 60, 4
    print(f"case bwd scale={scale} d={d}", flush=True)
    q, k, v = I.small_train_inputs(b, hq, hkv, d, P, L, 71 + d)
    do = I.small_grad_output(b, hq, d, P, L, 71 + d)
    q64, k64, v64, do64 = (to_np64(t) for t in (q, k, v, do))
    ref_o, ref_lse = O.attn(q64, k64, v64, P, L, B, scale=scale)
    od = torch.from_numpy(ref_o).to(torch.bfloat16).to(dev())
    lsed = torch.from_numpy(ref_lse).to(torch.float32).to(dev())
    lse_err = np.abs(to_np64(lsed) - ref_lse) + 1e-6
    dq, dk, dv = M.mars_attn_bwd(q.to(dev()), k.to(dev()), v.to(dev()), od, lsed, do.to(dev()), P, L, B,
                                 scale=scale)
    torch.cuda.synchronize()
    ref = O.attn_bwd(q64, k64, v64, do64, P, L, B, scale=scale)
    bnd = bwd_bounds(q64, k64, v64, do64, to_np64(od), lse_err, P, L, B, scale=scale)
    for name, g, r, bb in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref, bnd):
        check_bounded(to_np64(g), r, bb, f"{name} scale {scale} d{d}")


@pytest.mark.parametrize("scale", SCALES)
@pytest.mark.parametrize("noalloc", [False, True], ids=["ws", "noalloc"])
def test_decode_scale(scale, noalloc):
    """Cache chunks and window keys both at the given scale (a length of 1100 spans three
    cache chunks with a ragged last one)."""
    batch, hq, hkv, d, W, cap = 3, 28, 4, 128, 4, 1200
    lens = [1100, 7, 0]
    print(f"case decode scale={scale} noalloc={noalloc}", flush=True)
    s = I.DecodeShape("adhoc", batch, hq, hkv, d, W, cap, 0, cap, 8, 0.95, 0.5, 404)
    x = I.decode_inputs(s, with_logits=False)
    cache_len = torch.tensor(lens, dtype=torch.int32)
    args = (x.q_win.to(dev()), x.k_win.to(dev()), x.v_win.to(dev()), x.k_cache.to(dev()), x.v_cache.to(dev()),
            cache_len.to(dev()))
    out = M.mars_decode_step_noalloc(*args, scale=scale) if noalloc else M.mars_decode_step(*args, scale=scale)
    torch.cuda.synchronize()
    ref = O.decode(to_np64(x.q_win), to_np64(x.k_win), to_np64(x.v_win), to_np64(x.k_cache), to_np64(x.v_cache),
                   np.asarray(lens), scale=scale)
    check_close(to_np64(out), ref, f"decode scale {scale} noalloc={noalloc}")
