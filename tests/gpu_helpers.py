"""Shared helpers for the GPU parity tests (comparison bars and expected tile logs)."""
import numpy as np
import torch

from oracle import mars_oracle as O

# Bars from the method's stated tolerances for bf16 attention outputs.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
PMAX_ABS = 1e-5
TIE_ZONE = 1e-5


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
