"""Pins for the oracle's attention and decode (CPU only).

Independent anchors:
  * the MARS blog's separate-forward check: clean-stream outputs equal a plain causal
    forward over [prompt; x] bit for bit in float64 (scalar path), and to rounding on
    the BLAS path (checked against torch's float64 scaled_dot_product_attention);
  * B = 1: a masked position sees the clean prefix plus itself (MARS §3.3, first
    position of a block);
  * noisy block k equals a decode step whose cache holds [prompt; clean blocks < k]
    and whose window is block k (MARS Fig. 2, sliding-window inference);
  * W = 1 decode equals a textbook single-query AR step (the blog's "W=1 appends no
    mask slots");
  * closed forms: K = 0 gives the mean of the visible V; constant V gives that constant;
  * torch float64 SDPA with an explicit boolean mask on small shapes.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import mars_oracle as O


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def sdpa_ref(q, k, v, vis, scale):
    """torch float64 SDPA, q [b,N,Hq,D], k/v [b,N,Hkv,D], vis [R,N] bool (GQA by repeat)."""
    G = q.shape[2] // k.shape[2]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).repeat_interleave(G, dim=2).permute(0, 2, 1, 3).contiguous()
    vt = torch.from_numpy(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3).contiguous()
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(vis), scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("b,Hq,Hkv,D,P,L,B", [
    (1, 1, 1, 8, 3, 10, 3),
    (2, 4, 2, 16, 0, 12, 4),
    (1, 6, 2, 8, 5, 9, 1),
    (1, 2, 1, 4, 2, 7, 9),
])
def test_attn_matches_torch_sdpa(b, Hq, Hkv, D, P, L, B):
    N = P + 2 * L
    q, k, v = rand((b, N, Hq, D), 1), rand((b, N, Hkv, D), 2), rand((b, N, Hkv, D), 3)
    scale = 1 / math.sqrt(D)
    out, lse = O.attn(q, k, v, P, L, B)
    ref = sdpa_ref(q, k, v, O.mask_rules(P, L, B), scale)
    assert np.max(np.abs(out - ref)) <= 1e-12
    # LSE against scipy-free log-sum-exp written with torch
    G = Hq // Hkv
    vis = torch.from_numpy(O.mask_rules(P, L, B))
    for h in range(Hq):
        s = scale * torch.from_numpy(q[0, :, h]) @ torch.from_numpy(k[0, :, h // G]).T
        s = s.masked_fill(~vis, -math.inf)
        assert np.max(np.abs(torch.logsumexp(s, 1).numpy() - lse[0, h])) <= 1e-12


def test_clean_rows_bit_identical_to_causal_scalar():
    """fp64 scalar path: masked keys add exact zeros, so clean rows equal AR bit for bit."""
    P, L, B, D = 3, 8, 4, 5
    N = P + 2 * L
    q, k, v = rand((N, D), 4), rand((N, D), 5), rand((N, D), 6)
    scale = 1 / math.sqrt(D)
    vis = O.mask_rules(P, L, B)
    full = O.attn_scalar(q, k, v, vis, scale)
    n = P + L
    causal = np.tril(np.ones((n, n), dtype=bool))
    ar = O.attn_scalar(q[:n], k[:n], v[:n], causal, scale)
    assert np.array_equal(full[:n], ar)


def test_clean_rows_equal_causal_blas():
    b, Hq, Hkv, D, P, L, B = 2, 4, 2, 16, 9, 20, 4
    N = P + 2 * L
    q, k, v = rand((b, N, Hq, D), 7), rand((b, N, Hkv, D), 8), rand((b, N, Hkv, D), 9)
    out, _ = O.attn(q, k, v, P, L, B)
    n = P + L
    G = Hq // Hkv
    qt = torch.from_numpy(q[:, :n]).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k[:, :n]).repeat_interleave(G, 2).permute(0, 2, 1, 3).contiguous()
    vt = torch.from_numpy(v[:, :n]).repeat_interleave(G, 2).permute(0, 2, 1, 3).contiguous()
    ref = F.scaled_dot_product_attention(qt, kt, vt, is_causal=True).permute(0, 2, 1, 3).numpy()
    assert np.max(np.abs(out[:, :n] - ref)) <= 1e-12


def test_b1_masked_position_sees_clean_prefix_plus_itself():
    P, L, D = 4, 9, 6
    N = P + 2 * L
    q, k, v = rand((1, N, 1, D), 10), rand((1, N, 1, D), 11), rand((1, N, 1, D), 12)
    out, _ = O.attn(q, k, v, P, L, 1)
    scale = 1 / math.sqrt(D)
    for t0 in range(L):
        r = P + L + t0
        keys = list(range(P + t0)) + [r]
        s = np.array([scale * q[0, r, 0] @ k[0, j, 0] for j in keys])
        p = np.exp(s - s.max())
        ref = (p[:, None] * v[0, keys, 0]).sum(0) / p.sum()
        assert np.max(np.abs(out[0, r, 0] - ref)) <= 1e-13


def test_noisy_block_equals_decode_step():
    """Noisy block k (0-indexed) = decode with cache [0, P + kB) and window = block k."""
    P, L, B, D, Hq, Hkv = 3, 12, 4, 5, 2, 1
    N = P + 2 * L
    q, k, v = rand((1, N, Hq, D), 13), rand((1, N, Hkv, D), 14), rand((1, N, Hkv, D), 15)
    scale = 1 / math.sqrt(D)
    vis = O.mask_rules(P, L, B)
    for blk in range(L // B):
        rows = np.arange(P + L + blk * B, P + L + (blk + 1) * B)
        n = P + blk * B
        cap = N
        kc = np.zeros((1, Hkv, cap, D)); vc = np.zeros((1, Hkv, cap, D))
        kc[0, :, :n] = k[0, :n].transpose(1, 0, 2)
        vc[0, :, :n] = v[0, :n].transpose(1, 0, 2)
        dec = O.decode_scalar(q[:, rows], k[:, rows], v[:, rows], kc, vc, np.array([n]), scale)
        for h in range(Hq):
            full = O.attn_scalar(q[0, rows, h], k[0, :, 0], v[0, :, 0], vis[rows], scale)
            assert np.array_equal(full, dec[0, :, h])
        dec_blas = O.decode(q[:, rows], k[:, rows], v[:, rows], kc, vc, np.array([n]))
        assert np.max(np.abs(dec_blas - dec)) <= 1e-12


def test_decode_w1_is_textbook_ar_step():
    b, Hq, Hkv, D, cap = 3, 4, 2, 8, 20
    lens = np.array([0, 7, 20])
    q = rand((b, 1, Hq, D), 16); kw = rand((b, 1, Hkv, D), 17); vw = rand((b, 1, Hkv, D), 18)
    kc = rand((b, Hkv, cap, D), 19); vc = rand((b, Hkv, cap, D), 20)
    out = O.decode(q, kw, vw, kc, vc, lens)
    G = Hq // Hkv
    for bi in range(b):
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([kc[bi, g, :lens[bi]], kw[bi, :, g]])
            vals = np.concatenate([vc[bi, g, :lens[bi]], vw[bi, :, g]])
            ref = F.scaled_dot_product_attention(
                torch.from_numpy(q[bi, :, h])[None], torch.from_numpy(keys)[None],
                torch.from_numpy(vals)[None])[0].numpy()
            assert np.max(np.abs(out[bi, :, h] - ref)) <= 1e-12


def test_decode_matches_torch_with_window_mask():
    b, W, Hq, Hkv, D, cap = 2, 4, 6, 2, 8, 16
    lens = np.array([5, 16])
    q = rand((b, W, Hq, D), 21); kw = rand((b, W, Hkv, D), 22); vw = rand((b, W, Hkv, D), 23)
    kc = rand((b, Hkv, cap, D), 24); vc = rand((b, Hkv, cap, D), 25)
    out = O.decode(q, kw, vw, kc, vc, lens)
    assert np.max(np.abs(out - O.decode_scalar(q, kw, vw, kc, vc, lens, 1 / math.sqrt(D)))) <= 1e-12
    G = Hq // Hkv
    for bi in range(b):
        n = lens[bi]
        vis = np.zeros((W, n + W), dtype=bool)
        vis[:, :n] = True
        vis[:, n:] = np.tril(np.ones((W, W), dtype=bool))
        for h in range(Hq):
            keys = np.concatenate([kc[bi, h // G, :n], kw[bi, :, h // G]])
            vals = np.concatenate([vc[bi, h // G, :n], vw[bi, :, h // G]])
            ref = F.scaled_dot_product_attention(
                torch.from_numpy(q[bi, :, h]), torch.from_numpy(keys), torch.from_numpy(vals),
                attn_mask=torch.from_numpy(vis)).numpy()
            assert np.max(np.abs(out[bi, :, h] - ref)) <= 1e-12


def test_decode_empty_cache_first_row_is_own_value():
    q = rand((1, 3, 2, 4), 26); kw = rand((1, 3, 1, 4), 27); vw = rand((1, 3, 1, 4), 28)
    kc = np.zeros((1, 1, 4, 4)); vc = np.zeros((1, 1, 4, 4))
    out = O.decode(q, kw, vw, kc, vc, np.array([0]))
    assert np.array_equal(out[0, 0, 0], vw[0, 0, 0]) and np.array_equal(out[0, 0, 1], vw[0, 0, 0])


def test_closed_forms():
    P, L, B, D = 4, 10, 3, 6
    N = P + 2 * L
    q, v = rand((1, N, 2, D), 29), rand((1, N, 1, D), 30)
    out, lse = O.attn(q, np.zeros((1, N, 1, D)), v, P, L, B)
    vis = O.mask_rules(P, L, B)
    mean = (vis.astype(float) @ v[0, :, 0]) / vis.sum(1, keepdims=True)
    assert np.max(np.abs(out[0, :, 0] - mean)) <= 1e-13
    assert np.max(np.abs(lse[0, 0] - np.log(vis.sum(1)))) <= 1e-13
    c = np.full((1, N, 1, D), 0.375)
    out2, _ = O.attn(q, rand((1, N, 1, D), 31), c, P, L, B)
    assert np.max(np.abs(out2 - 0.375)) <= 1e-15


# ---------------------------------------------------------------------------
# Backward (gradients of the forward)
# ---------------------------------------------------------------------------

def _fd_grads(q, k, v, w, P, L, B, eps=1e-6):
    """Central differences of f = sum(O * w) with respect to every entry of q, k, v."""
    def f():
        return float(np.sum(O.attn(q, k, v, P, L, B)[0] * w))
    out = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + eps
            fp = f()
            x[idx] = old - eps
            fm = f()
            x[idx] = old
            g[idx] = (fp - fm) / (2 * eps)
        out.append(g)
    return out


@pytest.mark.parametrize("b,Hq,Hkv,D,P,L,B", [
    (1, 2, 1, 4, 3, 5, 2),     # GQA, ragged last block
    (2, 2, 2, 3, 0, 4, 4),     # no prompt, one block
    (1, 3, 1, 2, 2, 3, 1),     # B = 1
    (1, 1, 1, 3, 4, 2, 5),     # B > L
])
def test_attn_bwd_matches_finite_differences(b, Hq, Hkv, D, P, L, B):
    """The analytic gradients equal central differences of the forward (a scalar loss
    sum(O * W) with random W = dO), to the truncation error of the differences."""
    N = P + 2 * L
    q, k, v = rand((b, N, Hq, D), 1), rand((b, N, Hkv, D), 2), rand((b, N, Hkv, D), 3)
    w = rand((b, N, Hq, D), 4)
    dq, dk, dv = O.attn_bwd(q, k, v, w, P, L, B)
    fq, fk, fv = _fd_grads(q, k, v, w, P, L, B)
    for name, a, n in (("dq", dq, fq), ("dk", dk, fk), ("dv", dv, fv)):
        assert np.max(np.abs(a - n)) < 1e-7 * max(1.0, np.max(np.abs(n))), name


def test_attn_bwd_matches_torch_autograd():
    """torch float64 autograd through SDPA with the same explicit mask (library cross-check,
    GQA by repeating K/V, whose gradients are then summed back per KV head)."""
    b, Hq, Hkv, D, P, L, B = 2, 6, 2, 16, 7, 21, 4
    N = P + 2 * L
    q, k, v, do = rand((b, N, Hq, D), 11), rand((b, N, Hkv, D), 12), rand((b, N, Hkv, D), 13), rand((b, N, Hq, D), 14)
    dq, dk, dv = O.attn_bwd(q, k, v, do, P, L, B)
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(0, 2, 1, 3).requires_grad_(True)
    kt = torch.from_numpy(k).requires_grad_(True)
    vt = torch.from_numpy(v).requires_grad_(True)
    ke = kt.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    ve = vt.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vis = torch.from_numpy(O.mask_rules(P, L, B).astype(bool))
    o = F.scaled_dot_product_attention(qt, ke, ve, attn_mask=vis, scale=1.0 / math.sqrt(D))
    o.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
    assert np.max(np.abs(qt.grad.permute(0, 2, 1, 3).numpy() - dq)) < 1e-12
    assert np.max(np.abs(kt.grad.numpy() - dk)) < 1e-12
    assert np.max(np.abs(vt.grad.numpy() - dv)) < 1e-12


def test_attn_bwd_constant_v_closed_form():
    """Every key carries the same value vector c: O = c whatever P is, so dQ = dK = 0 and
    dV_j = sum_i P_ij dO_i (the column sums of P weight dO)."""
    b, Hq, Hkv, D, P, L, B = 1, 2, 1, 5, 4, 6, 3
    N = P + 2 * L
    q, k, do = rand((b, N, Hq, D), 21), rand((b, N, Hkv, D), 22), rand((b, N, Hq, D), 23)
    v = np.broadcast_to(rand((1, 1, 1, D), 24), (b, N, Hkv, D)).copy()
    dq, dk, dv = O.attn_bwd(q, k, v, do, P, L, B)
    assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12
    vis = O.mask_rules(P, L, B)
    want = np.zeros((N, D))
    for h in range(Hq):
        s = (q[0, :, h] @ k[0, :, 0].T) / math.sqrt(D)
        s = np.where(vis, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        want += p.T @ do[0, :, h]
    assert np.max(np.abs(dv[0, :, 0] - want)) < 1e-12


def test_attn_bwd_clean_rows_equal_causal_gradient():
    """With dO zero on the noisy stream, only clean and prompt rows carry gradient, and the
    gradients with respect to [prompt; x] equal those of plain causal attention over
    [prompt; x] (the noisy stream only reads clean keys, it never feeds them)."""
    b, Hq, Hkv, D, P, L, B = 1, 2, 1, 6, 5, 9, 3
    N, PL = P + 2 * L, P + L
    q, k, v, do = rand((b, N, Hq, D), 31), rand((b, N, Hkv, D), 32), rand((b, N, Hkv, D), 33), rand((b, N, Hq, D), 34)
    do[:, PL:] = 0.0
    dq, dk, dv = O.attn_bwd(q, k, v, do, P, L, B)
    causal = lambda P_, L_, B_, rr=None: np.tril(np.ones((PL, PL), dtype=bool))[rr if rr is not None else slice(None)]
    cq, ck, cv = O.attn_bwd(q[:, :PL], k[:, :PL], v[:, :PL], do[:, :PL], PL, 0, 1, mask_fn=causal)
    assert np.max(np.abs(dq[:, :PL] - cq)) < 1e-12
    assert np.max(np.abs(dk[:, :PL] - ck)) < 1e-12 and np.max(np.abs(dv[:, :PL] - cv)) < 1e-12
    assert np.max(np.abs(dq[:, PL:])) == 0.0 and np.max(np.abs(dk[:, PL:])) == 0.0


def test_attn_bwd_row_and_key_subsets():
    """Restricting dQ to some rows and dK/dV to some keys returns exactly those slices."""
    b, Hq, Hkv, D, P, L, B = 2, 4, 2, 8, 6, 10, 4
    N = P + 2 * L
    q, k, v, do = rand((b, N, Hq, D), 41), rand((b, N, Hkv, D), 42), rand((b, N, Hkv, D), 43), rand((b, N, Hq, D), 44)
    dq, dk, dv = O.attn_bwd(q, k, v, do, P, L, B)
    rows, keys = np.array([0, 5, 7, 17, 25]), np.array([1, 6, 16, 20, 25])
    sq, sk, sv = O.attn_bwd(q, k, v, do, P, L, B, rows=rows, keys=keys)
    assert np.max(np.abs(sq - dq[:, rows])) < 1e-13
    assert np.max(np.abs(sk - dk[:, keys])) < 1e-13 and np.max(np.abs(sv - dv[:, keys])) < 1e-13


# ---------------------------------------------------------------------------
# KV commit and cursor advance
# ---------------------------------------------------------------------------

def test_kv_commit_per_sample_and_batch_min():
    b, Hkv, cap, D, W = 3, 2, 10, 4, 4
    kc, vc = rand((b, Hkv, cap, D), 51), rand((b, Hkv, cap, D), 52)
    kw, vw = rand((b, W, Hkv, D), 53), rand((b, W, Hkv, D), 54)
    ln = np.array([0, 5, 8], dtype=np.int32)
    nacc = np.array([3, 1, 4], dtype=np.int32)
    k2, v2, l2, valid, over = O.kv_commit(kc, vc, ln, kw, vw, nacc)
    # sequence 0: rows 0..2 at 0..2; sequence 1: row 0 at 5; sequence 2: 8 + 4 > 10 -> nothing
    assert l2.tolist() == [3, 6, 8] and over.tolist() == [False, False, True]
    assert valid.tolist() == [0b111, 0b1, 0]
    assert np.array_equal(k2[0, :, 0:3], kw[0, 0:3].transpose(1, 0, 2))
    assert np.array_equal(v2[1, :, 5], vw[1, 0])
    untouched = np.ones((b, Hkv, cap), dtype=bool)
    untouched[0, :, 0:3] = False
    untouched[1, :, 5] = False
    assert np.array_equal(k2[untouched], kc[untouched]) and np.array_equal(v2[untouched], vc[untouched])
    # batch minimum: every sequence advances by min n = 1
    k3, v3, l3, valid3, over3 = O.kv_commit(kc, vc, ln, kw, vw, nacc, batch_min=True)
    assert l3.tolist() == [1, 6, 9] and valid3.tolist() == [1, 1, 1] and not over3.any()
    assert np.array_equal(k3[2, :, 8], kw[2, 0])


def test_kv_commit_then_decode_equals_decode_over_longer_cache():
    """Committing window rows 0..n-1 and decoding a new window equals one decode whose
    cache already held them (the cursor semantics the decode step relies on)."""
    b, Hq, Hkv, cap, D, W = 2, 4, 2, 16, 8, 3
    kc, vc = rand((b, Hkv, cap, D), 61), rand((b, Hkv, cap, D), 62)
    ln = np.array([4, 7], dtype=np.int32)
    kw, vw = rand((b, W, Hkv, D), 63), rand((b, W, Hkv, D), 64)
    k2, v2, l2, _, _ = O.kv_commit(kc, vc, ln, kw, vw, np.array([2, 3]))
    qn, kn, vn = rand((b, W, Hq, D), 65), rand((b, W, Hkv, D), 66), rand((b, W, Hkv, D), 67)
    got = O.decode(qn, kn, vn, k2, v2, l2)
    for bi in range(b):
        n = int(l2[bi])
        # reference: the same cache built by hand
        kref, vref = kc.copy(), vc.copy()
        m = n - int(ln[bi])
        kref[bi, :, ln[bi]:n] = kw[bi, :m].transpose(1, 0, 2)
        vref[bi, :, ln[bi]:n] = vw[bi, :m].transpose(1, 0, 2)
        ref = O.decode(qn[bi:bi + 1], kn[bi:bi + 1], vn[bi:bi + 1], kref[bi:bi + 1], vref[bi:bi + 1], l2[bi:bi + 1])
        assert np.array_equal(got[bi:bi + 1], ref)


# ---------------------------------------------------------------------------
# Right-shifted cross-entropy (Eq. 3 and Eq. 5)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("P,L,B", [(3, 8, 4), (0, 9, 4), (5, 6, 1), (2, 5, 8)])
def test_shifted_ce_term_counts_and_eq4(P, L, B):
    """Every response token has exactly one AR and one mask term (the first one none when
    there is no prompt), and the mask terms taken from clean rows are the block starts:
    their share is ceil(L/B)/L, Eq. 4's 1/B when B divides L."""
    tgt, war, wmask = O.shifted_ce_targets(P, L, B)
    n_tok = L - (1 if P == 0 else 0)
    assert war.sum() == n_tok and wmask.sum() == n_tok
    PL = P + L
    clean_mask = wmask[:PL].sum()
    assert clean_mask == -(-L // B) - (1 if P == 0 else 0)
    if P > 0 and L % B == 0:
        assert clean_mask / wmask.sum() == 1.0 / B
    # targets: clean row P-1+t -> t; noisy row PL+j -> j+1, never a block start
    for r in np.nonzero(tgt >= 0)[0]:
        if r < PL:
            assert tgt[r] == r - P + 1
        else:
            assert tgt[r] == r - PL + 1 and (r - PL + 1) % B != 0


def test_shifted_ce_uniform_logits_closed_form():
    P, L, B, V = 4, 8, 4, 37
    z = np.zeros((2, P + 2 * L, V))
    x = np.random.default_rng(3).integers(0, V, size=(2, L))
    lm, la, d = O.shifted_ce(z, x, P, L, B)
    assert np.allclose(la, L * math.log(V), rtol=0, atol=1e-12)
    assert np.allclose(lm, L * math.log(V), rtol=0, atol=1e-12)


def test_shifted_ce_matches_torch_cross_entropy_and_gradient():
    """torch float64 cross_entropy on the selected rows (library cross-check) and central
    differences of L_mask + L_AR for the gradient."""
    P, L, B, V = 2, 7, 3, 11
    rng = np.random.default_rng(9)
    z = rng.standard_normal((2, P + 2 * L, V))
    x = rng.integers(0, V, size=(2, L))
    lm, la, d = O.shifted_ce(z, x, P, L, B)
    tgt, war, wmask = O.shifted_ce_targets(P, L, B)
    zt = torch.from_numpy(z)
    for bi in range(2):
        for w, ref in ((war, la[bi]), (wmask, lm[bi])):
            rows = np.nonzero(w)[0]
            ce = F.cross_entropy(zt[bi, rows], torch.from_numpy(x[bi, tgt[rows]]), reduction="sum").item()
            assert abs(ce - ref) < 1e-12
    eps = 1e-6
    for (bi, r, v) in [(0, 1, 3), (1, P + L + 2, 7), (0, P + 3, 0), (1, P + 2 * L - 1, 5), (0, P + L + 1, 10)]:
        zp, zm = z.copy(), z.copy()
        zp[bi, r, v] += eps
        zm[bi, r, v] -= eps
        fp = sum(a.sum() for a in O.shifted_ce(zp, x, P, L, B)[:2])
        fm = sum(a.sum() for a in O.shifted_ce(zm, x, P, L, B)[:2])
        assert abs((fp - fm) / (2 * eps) - d[bi, r, v]) < 1e-7
