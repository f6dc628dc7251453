"""Shared helpers for the GPU parity tests (comparison bars and expected tile logs)."""
import numpy as np
import torch

from oracle import mars_oracle as O

# Bars from the method's stated tolerances for bf16 attention outputs.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
PMAX_ABS = 1e-5
TIE_ZONE = 1e-5
# Fixed accuracy targets beside the bounds derived from the kernels' roundings (those scale
# with the inputs; these do not): |LSE - LSE_exact| in nats on the workloads' input scales,
# and a gradient's max abs error against its own scale (max |ref|).
LSE_FIXED = 2e-2
GRAD_FIXED_REL = 2e-2
GRAD_FIXED_ABS = 1e-3


def lse_bound(q, k, scale=None):
    """Per-row bound [b, Hq, N] on |LSE_kernel - LSE_exact| (nats) for the bf16 kernel.

    Two roundings enter the kernel's log-sum-exp beyond fp32 accumulation:
      * every probability term is rounded to bf16 before it is summed, which moves log l
        by at most u = 2^-8 (the unit roundoff of bf16: an 8-bit significand, so
        round-to-nearest changes a value by at most 2^-8 of itself);
      * Q is multiplied by scale*log2(e) and rounded to bf16 once, which moves score j of
        row r by at most u * c * sum_i |q_ri| |k_ji| (log2 units; c = scale*log2(e)), and
        log-sum-exp moves by at most the largest score change.  The max is taken over
        every key (a superset of the visible ones).
    Plus 1e-5 for fp32 arithmetic.
    """
    qa, ka = np.abs(to_np64(q)), np.abs(to_np64(k))
    b, N, hq, d = qa.shape
    G = hq // ka.shape[2]
    c = (1.0 / np.sqrt(d) if scale is None else scale) * np.log2(np.e)
    u = 2.0 ** -8
    out = np.empty((b, hq, N))
    for bi in range(b):
        for h in range(hq):
            out[bi, h] = (qa[bi, :, h, :] @ ka[bi, :, h // G, :].T).max(axis=1)
    return u + np.log(2.0) * u * c * out + 1e-5


def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def to_np64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def check_close(got, ref, what, max_abs=O_MAX_ABS, mean_abs=O_MEAN_ABS):
    err = np.abs(np.asarray(got, dtype=np.float64) - ref)
    mx, mean = float(err.max()) if err.size else 0.0, float(err.mean()) if err.size else 0.0
    print(f"[{what}] max_abs={mx:.3e} mean_abs={mean:.3e}", flush=True)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert mx <= max_abs, f"{what}: max abs {mx} > {max_abs}"
    assert mean <= mean_abs, f"{what}: mean abs {mean} > {mean_abs}"
    return mx, mean


def expected_tilelog(P, L, B, G, row_block, key_block):
    """What the bf16 kernel must do per (row group, key group) of one (batch, kv head) pair.

    Rows are packed (position u // G); class 0 = no visible key, 2 = every key visible and the
    key group lies inside [0, N), 1 otherwise.  Derived from the oracle's dense mask.
    """
    N = P + 2 * L
    R = N * G
    nrg = -(-R // row_block)
    nkt = -(-N // key_block)
    vis = O.mask_rules(P, L, B)
    out = np.zeros((nrg, nkt), dtype=np.int8)
    for rg in range(nrg):
        pos = np.unique(np.arange(rg * row_block, min(R, (rg + 1) * row_block)) // G)
        rows = vis[pos]
        for kt in range(nkt):
            blk = rows[:, kt * key_block:min(N, (kt + 1) * key_block)]
            if blk.any():
                out[rg, kt] = 2 if (blk.all() and (kt + 1) * key_block <= N) else 1
    return out


def sample_rows(P, L, B, n_random, seed):
    """Boundary positions plus random ones (the sampled-output parity at full size)."""
    N = P + 2 * L
    rng = np.random.default_rng(seed)
    fixed = [0, max(P - 1, 0), P, P + 1, P + L - 1, P + L, P + L + 1, P + L + B - 1, P + L + B,
             N - B - 1, N - B, N - 2, N - 1, P + L // 2, P + L + L // 2]
    rows = set(r for r in fixed if 0 <= r < N)
    rows.update(rng.integers(0, N, size=n_random).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def bwd_bounds(q, k, v, do, o_in, lse_err, P, L, B, rows=None, keys=None, scale=None):
    """Per-element bounds on |grad_kernel - grad_exact| for the bf16 backward.

    q, k, v, do: float64 copies of the bf16 inputs; o_in: the O handed to the kernel;
    lse_err: [b, Hq, N] bound on |LSE_in - LSE_exact| (nats).  Sources of error, each bounded
    by its largest effect (u = 2^-8, bf16's unit roundoff):
      * the scores round one operand times c = scale*log2 e to bf16 (Q in dQ, as the forward
        does; K in dK/dV): score (i, j) moves by at most u*c*sum_d |q_id||k_jd| (log2 units),
        so P_ij by a relative 2^(u c m_i) - 1 with m_i the max over keys; the LSE input adds
        e^lse_err - 1;
      * D_i = sum dO.O from the given O: |dD_i| <= sum_d |dO_id||O_in - O_exact|_id;
      * P (for dV) and dS (for dQ, dK) are rounded to bf16 (u each); at head_dim 128 the dK
        side forms dS from the bf16 P the dV side uses (one more u on dS);
      * fp32 accumulation over n terms: n*2^-24 of the sum of absolute terms;
      * the bf16 output rounding: u |grad|.
    Returns (bq [b,R,Hq,D], bk [b,K,Hkv,D], bv [b,K,Hkv,D]) for rows / keys (all by default).
    """
    b, N, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    c = scale * np.log2(np.e)
    u = 2.0 ** -8
    rows = np.arange(N) if rows is None else np.asarray(rows)
    keys = np.arange(N) if keys is None else np.asarray(keys)
    cols = np.zeros(N, dtype=bool)
    cols[keys] = True
    vis_all = O.mask_rules(P, L, B)
    krows = np.nonzero((vis_all & cols[None, :]).any(axis=1))[0]
    gam = N * 2.0 ** -24
    bq = np.zeros((b, len(rows), Hq, D))
    bk = np.zeros((b, len(keys), Hkv, D))
    bv = np.zeros((b, len(keys), Hkv, D))
    for bi in range(b):
        for h in range(Hq):
            g = h // G
            for rr, want_q in ((rows, True), (krows, False)):
                if len(rr) == 0:
                    continue
                vis = vis_all[rr]
                qa = q[bi, rr, h]
                s = scale * (qa @ k[bi, :, g].T)
                s = np.where(vis, s, -np.inf)
                e = np.exp(s - s.max(axis=1, keepdims=True))
                p = e / e.sum(axis=1, keepdims=True)
                o = p @ v[bi, :, g]
                dO = do[bi, rr, h]
                x = dO @ v[bi, :, g].T - np.sum(dO * o, axis=1, keepdims=True)      # dP - D
                m = (np.abs(qa) @ np.abs(k[bi, :, g]).T).max(axis=1)
                rel = 2.0 ** (u * c * m) - 1.0 + np.expm1(lse_err[bi, h, rr])       # relative error of P
                eD = np.sum(np.abs(dO) * np.abs(o_in[bi, rr, h] - o), axis=1)        # |dD|
                rel, eD = rel[:, None], eD[:, None]
                ds = p * x
                dds = p * (rel * np.abs(x) + (1 + rel) * eD) + u * (1 + rel) * p * (np.abs(x) + eD) \
                    + gam * p * (np.abs(dO) @ np.abs(v[bi, :, g]).T)
                if want_q:
                    dq = scale * (ds @ k[bi, :, g])
                    bq[bi, :, h] = scale * (dds @ np.abs(k[bi, :, g])) * (1 + gam) \
                        + gam * scale * (np.abs(ds) @ np.abs(k[bi, :, g])) + u * np.abs(dq) + 1e-6
                else:
                    ddk = dds + (u * (1 + rel) * p * (np.abs(x) + eD) if D == 128 else 0.0)
                    pk, dsk, ddsk = p[:, keys], ds[:, keys], ddk[:, keys]
                    relv = rel + u * (1 + rel)
                    bv[bi, :, g] += (pk * relv).T @ np.abs(dO) + gam * (pk.T @ np.abs(dO))
                    bk[bi, :, g] += scale * ((ddsk + u * np.abs(dsk)).T @ np.abs(qa)) \
                        + gam * scale * (np.abs(dsk).T @ np.abs(qa))
    # output rounding of dK / dV (relative to the exact value, bounded by the sums above)
    return bq, bk, bv


def check_bounded(got, ref, bound, what, extra_rel=2.0 ** -8, fixed=True):
    """|got - ref| <= bound + extra_rel*|ref| elementwise (extra_rel: output rounding); with
    ``fixed``, also max |got - ref| <= GRAD_FIXED_REL * max |ref| + GRAD_FIXED_ABS."""
    got = np.asarray(got, dtype=np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    tol = bound + extra_rel * np.abs(ref) + 1e-6
    ratio = float(np.max(err / tol)) if err.size else 0.0
    mx, scale = (float(err.max()), float(np.abs(ref).max())) if err.size else (0.0, 0.0)
    print(f"[{what}] max_abs={mx:.3e} max|ref|={scale:.3e} max err/bound={ratio:.3f}", flush=True)
    assert ratio <= 1.0, f"{what}: error exceeds its bound (ratio {ratio:.3f})"
    if fixed:
        assert mx <= GRAD_FIXED_REL * scale + GRAD_FIXED_ABS, f"{what}: max abs {mx} beyond the fixed target"
    return ratio


def expected_tilelog_intervals(P, L, B, G, row_block, key_block):
    """:func:`expected_tilelog` built from the oracle's two-interval row encoding instead of
    the dense mask, so it scales to long layouts (N = 15360 and beyond).

    Row r sees [0, hi1) and [lo2, r] (oracle ``row_intervals``).  A key group [kb, ke) with
    its in-range part [kb, min(ke, N)) is visited by a row group iff some row of the group
    sees a key of it, and needs no element mask iff every row sees every key of it and
    ke <= N.  The two intervals of a row never touch when both are non-empty (L >= 1 puts
    the clean stream between them), so "every key" is "inside one interval".
    """
    N = P + 2 * L
    R = N * G
    nrg = -(-R // row_block)
    nkt = -(-N // key_block)
    kb = np.arange(nkt, dtype=np.int64) * key_block
    ke = np.minimum(kb + key_block, N)                # in-range end
    out = np.zeros((nrg, nkt), dtype=np.int8)
    for rg in range(nrg):
        pos = np.unique(np.arange(rg * row_block, min(R, (rg + 1) * row_block)) // G)
        hi1, lo2 = O.row_intervals(P, L, B, pos)
        r = pos[:, None]
        hi1, lo2 = hi1[:, None], lo2[:, None]
        any_ = (kb[None, :] < hi1) | (np.maximum(kb[None, :], lo2) <= np.minimum(ke[None, :] - 1, r))
        all_ = (ke[None, :] <= hi1) | ((kb[None, :] >= lo2) & (ke[None, :] - 1 <= r))
        vis = any_.any(axis=0)
        full = all_.all(axis=0) & (kb + key_block <= N)
        out[rg] = np.where(vis, np.where(full, 2, 1), 0)
    return out


def oracle_attn_slices(q, k, v, P, L, B, pairs, threads=None):
    """The oracle's attention for the (batch, query head) slices in ``pairs``, one slice per
    task on a thread pool (the oracle's large NumPy operations release the GIL; BLAS is held
    to one thread per task).  q/k/v: float64 arrays [b, N, H, D].
    Returns {(b, h): (O [N, D], LSE [N])}."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    G = q.shape[2] // k.shape[2]

    def one(bh):
        bi, h = bh
        o, lse = O.attn(q[bi:bi + 1, :, h:h + 1], k[bi:bi + 1, :, h // G:h // G + 1],
                        v[bi:bi + 1, :, h // G:h // G + 1], P, L, B)
        return bh, (o[0, :, 0], lse[0, 0])

    n = threads or min(16, max(1, (__import__("os").cpu_count() or 2)))
    with threadpool_limits(1), ThreadPoolExecutor(n) as ex:
        return dict(ex.map(one, list(pairs)))


def lse_bound_slices(q, k, pairs, scale=None, threads=None):
    """:func:`lse_bound` per (batch, query head) slice on a thread pool: {(b, h): bound [N]}."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    qa, ka = np.abs(q), np.abs(k)
    b, N, hq, d = qa.shape
    G = hq // ka.shape[2]
    c = (1.0 / np.sqrt(d) if scale is None else scale) * np.log2(np.e)
    u = 2.0 ** -8

    def one(bh):
        bi, h = bh
        m = np.empty(N)
        for r0 in range(0, N, 2048):
            m[r0:r0 + 2048] = (qa[bi, r0:r0 + 2048, h, :] @ ka[bi, :, h // G, :].T).max(axis=1)
        return bh, u + np.log(2.0) * u * c * m + 1e-5

    n = threads or min(16, max(1, (__import__("os").cpu_count() or 2)))
    with threadpool_limits(1), ThreadPoolExecutor(n) as ex:
        return dict(ex.map(one, list(pairs)))


def tie_zone_width(gate_kernel, gate64, tau):
    """Half-width of the band around tau inside which the kernel's decision may differ from
    the oracle's: the largest measured |gate_kernel - gate_oracle| over all rows plus the
    rounding of tau to fp32 (the kernel compares fp32 values).  A row farther from tau than
    this is decided the same way on both sides."""
    err = float(np.max(np.abs(np.asarray(gate_kernel, dtype=np.float64) - gate64))) if np.size(gate64) else 0.0
    return err + abs(float(np.float32(tau)) - tau)


def tie_zone_sequences(gate64, tau, width=TIE_ZONE):
    """Sequences whose acceptance count depends on a row whose gate value (the oracle's pmax or
    margin) lies within `width` of tau: the rows that decide n are the leading run of rows
    with gate >= tau and the first row after it; a later row cannot change n.  With tau >= 1
    exactly one token is accepted whatever the rows hold, so nothing is in the zone."""
    gate64 = np.asarray(gate64, dtype=np.float64)
    b, W = gate64.shape
    tie = np.zeros(b, dtype=bool)
    if tau >= 1.0:
        return tie
    for bi in range(b):
        run = 0
        while run < W and gate64[bi, run] >= tau:
            run += 1
        deciding = gate64[bi, :min(run + 1, W)]
        tie[bi] = bool(np.any(np.abs(deciding - tau) <= width))
    return tie
