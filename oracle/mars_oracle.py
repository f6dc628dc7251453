"""Plain fp64 CPU oracle for MARS structured-mask attention, decode step and acceptance.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, links or runs this
module: only the tests, the smoke check and the bench's ``cpu_baseline`` leg may.
It shares no code with the HIP library and imports nothing from it.

Every function is the plain definition written out, in float64, with no blocking,
fusion or reordering beyond what the definition states.  Sources (cited by page
title and section):

* [MARS] "MARS: Enabling Autoregressive Models Multi-Token Generation"
  (arXiv 2604.07023): §3.2 Eq. 1 (noisy copy), Eq. 2 (attention mask over
  z = [x; x~]), Fig. 2 (mask for L=8, B=4; sliding-window inference), §3.3 Eq. 4.
* [BLOG] MARS author blog post (xalp.net, "mars"), section "Inference: a knob,
  not a mode switch" (left-to-right commit while confidence >= tau, tau = 1.0 is
  exact AR) and "Batching is where methods like this usually die" (W = 1 appends
  no mask slots).
* [TRENDS] aitrends.kr summary of MARS, inference paragraph (at least one token
  is always accepted).
* [BLOG] section "Inference: a knob, not a mode switch", second finding: a margin
  gate (how far the top token is ahead, rather than how confident it is); and
  "Batching is where methods like this usually die": the block-level KV cache that
  advances at the batch-minimum acceptance, and the deferred-KV sampler with
  per-sample cursors and a cache-validity bitmask.

Readings taken where the pages are silent (each is listed in the design notes):

* The prompt is a causal prefix in front of [x; x~]: prompt rows see prompt keys
  up to themselves; clean and noisy rows see every prompt key; nothing in the
  prompt sees the response; block indices count from the first response token.
* Intra-block attention is self-inclusive (Eq. 2 states j <= i).
* GQA: query head h reads KV head h // (Hq / Hkv).
* Acceptance uses the temperature-1 softmax over the full vocabulary; the argmax
  tie rule is "lowest index"; tau >= 1 accepts exactly one token.
* KV commit: the accepted window rows 0..n-1 of a sequence are appended to its cache
  at its cursor, and the cursor advances by n; the per-sample policy uses each
  sequence's own n, the batch-minimum policy min over the batch for every sequence;
  a sequence whose cache cannot hold n more rows commits none and reports it; the
  validity bitmask of a sequence has bit i set iff window row i was committed.
* Training loss (MARS §3.2 Eq. 3, §3.3 Eq. 5, logits right-shifted as in AR: the logit
  row of position p predicts the token at p + 1): L_AR takes response token x_t from
  the clean row before it (the last prompt row for t = 0; none if there is no prompt);
  L_mask takes x_t from the noisy row before it inside its block, and the first token
  of a block, whose only fully clean context is the clean prefix (§3.3: position 1 of a
  block is exactly an AR prediction; Eq. 4's 1/B), from the same clean row as L_AR.
  Losses are sums of -log softmax(row)[target] (natural log).
* The margin gate's margin is the top-1 minus the top-2 probability of that softmax,
  where top-2 is the second largest entry of the row counted with multiplicity (a
  tied maximum gives margin 0); it commits the same way as the probability gate.

Parity status: every public function here is pinned by a ``-m "not gpu"`` test
(brute-force rule enumeration, the Fig. 2 matrix, closed forms, invariants and
library cross-checks); none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "block_index",
    "mask_rules_scalar",
    "mask_rules",
    "mask_intervals",
    "row_intervals",
    "mask_nnz",
    "attn",
    "attn_scalar",
    "attn_bwd",
    "tile_map",
    "tile_map_rules",
    "visible_tile_elems",
    "decode",
    "decode_scalar",
    "accept_rows",
    "accept",
    "accept_scalar",
    "accept_margin",
    "accept_margin_scalar",
    "kv_commit",
    "shifted_ce_targets",
    "shifted_ce",
]


# ---------------------------------------------------------------------------
# Mask (MARS §3.2, Eq. 2, plus the prompt reading)
# ---------------------------------------------------------------------------

def block_index(t, B):
    """beta(t) = ceil(t / B) for a 1-indexed position t inside either stream ([MARS] §3.2)."""
    return -(-np.asarray(t) // B)


def _eq2_visible(i, j, L, B):
    """Eq. 2 of [MARS] §3.2 on 1-indexed z-positions i (query), j (key), 1 <= i, j <= 2L.

    True where M_ij = 0, False where M_ij = -inf.  Works elementwise on arrays.
    """
    i = np.asarray(i)
    j = np.asarray(j)
    clean_causal = (i <= L) & (j <= L) & (j <= i)
    noisy_intra = (i > L) & (j > L) & (block_index(i - L, B) == block_index(j - L, B)) & (j <= i)
    # block_index of a non-positive argument is never used: the & masks it out.
    noisy_to_clean = (i > L) & (j <= L) & (block_index(j, B) < block_index(np.maximum(i - L, 1), B))
    return clean_causal | noisy_intra | noisy_to_clean


def mask_rules_scalar(P, L, B):
    """Dense visibility over [prompt; x; x~] by explicit loops (tiny shapes only).

    Positions are 1-indexed as in [MARS] §3.2.  Returns uint8 [N, N], N = P + 2L,
    1 = visible.  The prompt reading: prompt rows are causal over the prompt; every
    response row (clean or noisy) sees the whole prompt; the prompt sees no response.
    """
    N = P + 2 * L
    m = np.zeros((N, N), dtype=np.uint8)
    for a in range(1, N + 1):
        for c in range(1, N + 1):
            if a <= P:
                vis = c <= a
            elif c <= P:
                vis = True
            else:
                i, j = a - P, c - P
                if i <= L and j <= L:
                    vis = j <= i
                elif i > L and j > L:
                    vis = (math.ceil((i - L) / B) == math.ceil((j - L) / B)) and j <= i
                elif i > L and j <= L:
                    vis = math.ceil(j / B) < math.ceil((i - L) / B)
                else:
                    vis = False
            m[a - 1, c - 1] = 1 if vis else 0
    return m


def mask_rules(P, L, B, rows=None):
    """Vectorised form of :func:`mask_rules_scalar` (same rules, Eq. 2 case by case).

    ``rows``: optional 0-indexed query positions to materialise (default: all N).
    Returns bool [len(rows), N].
    """
    N = P + 2 * L
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    a = rows[:, None] + 1          # 1-indexed query position in [prompt; z]
    c = np.arange(1, N + 1)[None, :]
    prompt_row = a <= P
    prompt_key = c <= P
    i = a - P
    j = c - P
    resp = (~prompt_row) & (~prompt_key)
    vis = np.where(prompt_row, c <= a, False)
    vis |= (~prompt_row) & prompt_key
    # Eq. 2 evaluated only where both positions are response positions.
    ii = np.where(resp, i, 1)
    jj = np.where(resp, j, 1)
    vis |= resp & _eq2_visible(ii, jj, L, B)
    return vis


def row_intervals(P, L, B, rows=None):
    """Two-interval encoding of each row's visible keys (0-indexed, half-open).

    Row r sees keys [0, hi1) and [lo2, r + 1).  For prompt and clean rows the second
    interval is empty (lo2 = r + 1) and hi1 = r + 1.  A noisy row at response offset
    t0 = r - P - L, block k = t0 // B, sees [0, P + kB) (prompt plus the clean tokens
    of earlier blocks) and [P + L + kB, r] (its own block up to itself).
    """
    N = P + 2 * L
    r = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    noisy = r >= P + L
    k = np.where(noisy, (r - P - L) // B, 0)
    hi1 = np.where(noisy, P + k * B, r + 1)
    lo2 = np.where(noisy, P + L + k * B, r + 1)
    return hi1, lo2


def mask_intervals(P, L, B, rows=None):
    """Dense bool mask built from :func:`row_intervals` (independent second encoding)."""
    N = P + 2 * L
    r = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    hi1, lo2 = row_intervals(P, L, B, r)
    j = np.arange(N)[None, :]
    return (j < hi1[:, None]) | ((j >= lo2[:, None]) & (j <= r[:, None]))


def mask_nnz(P, L, B):
    """Number of visible (query, key) pairs, by summing the per-row interval lengths."""
    hi1, lo2 = row_intervals(P, L, B)
    r = np.arange(P + 2 * L)
    return int(np.sum(hi1) + np.sum(r + 1 - lo2))


# ---------------------------------------------------------------------------
# Training-layout attention: O = softmax(scale * Q K^T + M) V
# ---------------------------------------------------------------------------

def _gqa_group(Hq, Hkv):
    if Hkv <= 0 or Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    return Hq // Hkv


def attn(q, k, v, P, L, B, scale=None, rows=None, row_chunk=1024, mask_fn=mask_rules):
    """Masked attention over [prompt; x; x~] in float64.

    q: [b, N, Hq, D]; k, v: [b, N, Hkv, D] (any float dtype; upcast to float64).
    Query head h uses KV head h // (Hq/Hkv).  ``rows`` restricts the output to those
    0-indexed query positions.  Returns (O [b, R, Hq, D] float64, LSE [b, Hq, R]).
    The mask is materialised explicitly (``mask_fn``); masked scores are -inf; then
    m = rowmax, p = exp(S - m), O = p V / sum p, LSE = m + ln sum p.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b, N, Hq, D = q.shape
    Hkv = k.shape[2]
    assert N == P + 2 * L and k.shape == (b, N, Hkv, D) and v.shape == k.shape
    G = _gqa_group(Hq, Hkv)
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(D)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    out = np.zeros((b, R, Hq, D))
    lse = np.zeros((b, Hq, R))
    for c0 in range(0, R, row_chunk):
        rr = rows[c0:c0 + row_chunk]
        vis = mask_fn(P, L, B, rr)
        for bi in range(b):
            for h in range(Hq):
                g = h // G
                s = scale * (q[bi, rr, h, :] @ k[bi, :, g, :].T)
                s = np.where(vis, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                den = p.sum(axis=1, keepdims=True)
                out[bi, c0:c0 + len(rr), h, :] = (p @ v[bi, :, g, :]) / den
                lse[bi, h, c0:c0 + len(rr)] = m[:, 0] + np.log(den[:, 0])
    return out, lse


def attn_bwd(q, k, v, do, P, L, B, scale=None, rows=None, keys=None, mask_fn=mask_rules):
    """Gradients of :func:`attn` with respect to q, k and v for an upstream gradient dO.

    Training needs the gradient of this exact forward ([MARS] §3.2-3.3: the loss of
    Eq. 3/5 is taken through the Eq. 2 attention).  For one (batch, head), with
    S = scale Q K^T + M, P = softmax(S) row-wise and O = P V, the chain rule through
    the row softmax gives, in float64:

        D_i  = sum_d dO_id O_id                      (= sum_j P_ij dP_ij)
        dP   = dO V^T,   dS = P o (dP - D)           (masked entries: P = 0, dS = 0)
        dQ   = scale dS K,   dK = scale dS^T Q,   dV = P^T dO

    and dK, dV of KV head g are summed over the query heads h with h // G = g.
    ``rows`` restricts dQ to those query positions; ``keys`` restricts dK and dV to
    those key positions (only the rows that see one of them are evaluated, each
    with its full softmax).  Returns (dq [b, R, Hq, D], dk [b, K, Hkv, D],
    dv [b, K, Hkv, D]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    b, N, Hq, D = q.shape
    Hkv = k.shape[2]
    assert N == P + 2 * L and k.shape == (b, N, Hkv, D) and v.shape == k.shape and do.shape == q.shape
    G = _gqa_group(Hq, Hkv)
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(D)
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(N) if keys is None else np.asarray(keys, dtype=np.int64)
    dq = np.zeros((b, len(rows), Hq, D))
    dk = np.zeros((b, len(keys), Hkv, D))
    dv = np.zeros((b, len(keys), Hkv, D))

    def probs(bi, h, rr):
        """Row-normalised P and O for query rows rr of (bi, h)."""
        g = h // G
        vis = mask_fn(P, L, B, rr)
        s = scale * (q[bi, rr, h, :] @ k[bi, :, g, :].T)
        s = np.where(vis, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        p = e / e.sum(axis=1, keepdims=True)
        return p, p @ v[bi, :, g, :]

    # Query rows that see at least one requested key (the only rows with dS in those columns).
    kr = np.unique(keys)
    cols = np.zeros(N, dtype=bool)
    cols[kr] = True
    krows = np.array([i for i in range(N) if np.any(mask_fn(P, L, B, np.array([i]))[0] & cols)], dtype=np.int64)
    for bi in range(b):
        for h in range(Hq):
            g = h // G
            if len(rows):
                p, o = probs(bi, h, rows)
                dO = do[bi, rows, h, :]
                Dv = np.sum(dO * o, axis=1, keepdims=True)
                ds = p * (dO @ v[bi, :, g, :].T - Dv)
                dq[bi, :, h, :] = scale * (ds @ k[bi, :, g, :])
            if len(krows):
                p, o = probs(bi, h, krows)
                dO = do[bi, krows, h, :]
                Dv = np.sum(dO * o, axis=1, keepdims=True)
                pk = p[:, keys]
                ds = pk * (dO @ v[bi, keys, g, :].T - Dv)
                dk[bi, :, g, :] += scale * (ds.T @ q[bi, krows, h, :])
                dv[bi, :, g, :] += pk.T @ dO
    return dq, dk, dv


def attn_scalar(q, k, v, vis, scale):
    """Single-head masked attention by explicit loops in key order (tiny shapes only).

    q: [R, D], k, v: [N, D], vis: bool [R, N].  Python floats (IEEE double), keys
    visited in increasing index order; a masked key contributes exactly +0.0 to the
    running sums.  Used for the bit-exact invariants.
    """
    R, D = len(q), len(q[0])
    N = len(k)
    out = [[0.0] * D for _ in range(R)]
    for i in range(R):
        s = [0.0] * N
        m = -math.inf
        for j in range(N):
            if vis[i][j]:
                acc = 0.0
                for d in range(D):
                    acc += float(q[i][d]) * float(k[j][d])
                s[j] = scale * acc
                m = max(m, s[j])
        den = 0.0
        num = [0.0] * D
        for j in range(N):
            p = math.exp(s[j] - m) if vis[i][j] else 0.0
            den += p
            for d in range(D):
                num[d] += p * float(v[j][d])
        out[i] = [x / den for x in num]
    return np.array(out, dtype=np.float64)


def tile_map(vis, bm, bn):
    """Per (q-tile, k-tile) class on a bm x bn grid: 0 all masked, 2 all visible, 1 mixed.

    Only in-range elements count (ragged last tiles are classified on what they hold).
    ``vis``: bool [N, N].  Returns int8 [ceil(N/bm), ceil(N/bn)].
    """
    N0, N1 = vis.shape
    T0, T1 = -(-N0 // bm), -(-N1 // bn)
    out = np.zeros((T0, T1), dtype=np.int8)
    for a in range(T0):
        for c in range(T1):
            blk = vis[a * bm:(a + 1) * bm, c * bn:(c + 1) * bn]
            if blk.all():
                out[a, c] = 2
            elif blk.any():
                out[a, c] = 1
    return out


def tile_map_rules(P, L, B, bm, bn):
    """:func:`tile_map` of the Eq. 2 mask, built one q-tile row band at a time.

    Same classification as ``tile_map(mask_rules(P, L, B), bm, bn)`` without holding
    the N x N mask (the long layouts have N = 15360).
    """
    N = P + 2 * L
    T0 = -(-N // bm)
    bands = []
    for a in range(T0):
        rows = np.arange(a * bm, min(N, (a + 1) * bm))
        bands.append(tile_map(mask_rules(P, L, B, rows), bm, bn))
    return np.concatenate(bands, axis=0) if bands else np.zeros((0, 0), dtype=np.int8)


def visible_tile_elems(P, L, B, bm, bn):
    """In-range (query, key) elements of the tiles that are not fully masked.

    4 * D * this * batch * Hq is the "visible-tile" FLOP count of a forward on a
    bm x bn grid (QK^T and PV, 2 FLOP per multiply-add each).
    """
    N = P + 2 * L
    tm = tile_map_rules(P, L, B, bm, bn)
    h = np.minimum(bm, N - bm * np.arange(tm.shape[0]))
    w = np.minimum(bn, N - bn * np.arange(tm.shape[1]))
    return int(np.sum((tm > 0) * np.outer(h, w)))


# ---------------------------------------------------------------------------
# Sliding-window decode step ([MARS] Fig. 2 right; [BLOG] inference section)
# ---------------------------------------------------------------------------

def decode(q_win, k_win, v_win, k_cache, v_cache, cache_len, scale=None):
    """Attention of W window rows against a per-sequence KV cache plus the window.

    q_win [b, W, Hq, D]; k_win, v_win [b, W, Hkv, D]; k_cache, v_cache
    [b, Hkv, cap, D]; cache_len [b] (0 <= len <= cap).  Window row i of sequence bi
    attends to cache positions [0, len_bi) followed by window rows 0..i (causal,
    self-inclusive, as within a noisy block of Eq. 2).  Returns O [b, W, Hq, D] float64.
    """
    q_win = np.asarray(q_win, dtype=np.float64)
    k_win = np.asarray(k_win, dtype=np.float64)
    v_win = np.asarray(v_win, dtype=np.float64)
    k_cache = np.asarray(k_cache, dtype=np.float64)
    v_cache = np.asarray(v_cache, dtype=np.float64)
    b, W, Hq, D = q_win.shape
    Hkv = k_win.shape[2]
    G = _gqa_group(Hq, Hkv)
    if scale is None or scale == 0:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros((b, W, Hq, D))
    for bi in range(b):
        n = int(cache_len[bi])
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([k_cache[bi, g, :n, :], k_win[bi, :, g, :]], axis=0)
            vals = np.concatenate([v_cache[bi, g, :n, :], v_win[bi, :, g, :]], axis=0)
            s = scale * (q_win[bi, :, h, :] @ keys.T)          # [W, n + W]
            vis = np.ones_like(s, dtype=bool)
            for i in range(W):
                vis[i, n + i + 1:] = False
            s = np.where(vis, s, -np.inf)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            out[bi, :, h, :] = (p @ vals) / p.sum(axis=1, keepdims=True)
    return out


def decode_scalar(q_win, k_win, v_win, k_cache, v_cache, cache_len, scale):
    """Loop form of :func:`decode` built on :func:`attn_scalar` (tiny shapes only)."""
    b, W, Hq, D = q_win.shape
    Hkv = k_win.shape[2]
    G = _gqa_group(Hq, Hkv)
    out = np.zeros((b, W, Hq, D))
    for bi in range(b):
        n = int(cache_len[bi])
        for h in range(Hq):
            g = h // G
            keys = np.concatenate([k_cache[bi, g, :n, :], k_win[bi, :, g, :]], axis=0)
            vals = np.concatenate([v_cache[bi, g, :n, :], v_win[bi, :, g, :]], axis=0)
            vis = [[j < n + i + 1 for j in range(n + W)] for i in range(W)]
            out[bi, :, h, :] = attn_scalar(q_win[bi, :, h, :], keys, vals, vis, scale)
    return out


# ---------------------------------------------------------------------------
# Confidence-threshold acceptance ([BLOG] inference section; [TRENDS] inference)
# ---------------------------------------------------------------------------

def accept_rows(logits):
    """Per row of logits [..., V]: (argmax with lowest-index ties, top-1 softmax probability).

    Temperature-1 softmax over the full vocabulary, in float64:
    m = max, token = min{v : l_v = m}, S = sum exp(l - m), pmax = 1 / S.
    """
    x = np.asarray(logits, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    token = np.argmax(x == m, axis=-1)          # first index attaining the max
    S = np.exp(x - m).sum(axis=-1)
    return token.astype(np.int32), 1.0 / S


def accept(logits, tau):
    """Acceptance over a window: logits [b, W, V] -> (tokens [b, W], pmax [b, W], n [b]).

    Commit window positions left to right while pmax >= tau, stop at the first one
    below tau, and always commit at least one.  tau >= 1 is the exact AR fallback
    and commits exactly one.
    """
    tokens, pmax = accept_rows(logits)
    b, W = pmax.shape
    n = np.zeros(b, dtype=np.int32)
    for bi in range(b):
        if tau >= 1.0:
            n[bi] = 1
            continue
        run = 0
        while run < W and pmax[bi, run] >= tau:
            run += 1
        n[bi] = max(1, run)
    return tokens, pmax, n


def accept_scalar(logits, tau):
    """Loop form of :func:`accept` with compensated summation (tiny vocabularies)."""
    x = np.asarray(logits, dtype=np.float64)
    b, W, V = x.shape
    tokens = np.zeros((b, W), dtype=np.int32)
    pmax = np.zeros((b, W))
    n = np.zeros(b, dtype=np.int32)
    for bi in range(b):
        for i in range(W):
            row = [float(t) for t in x[bi, i]]
            best, arg = row[0], 0
            for vi in range(1, V):
                if row[vi] > best:
                    best, arg = row[vi], vi
            tokens[bi, i] = arg
            pmax[bi, i] = 1.0 / math.fsum(math.exp(t - best) for t in row)
        cnt = 0
        if tau < 1.0:
            for i in range(W):
                if pmax[bi, i] >= tau:
                    cnt += 1
                else:
                    break
        n[bi] = max(1, cnt)
    return tokens, pmax, n


def accept_margin(logits, tau):
    """Margin-gate acceptance: logits [b, W, V] -> (tokens, pmax, margin, n).

    Per row, with l1 >= l2 the two largest entries (with multiplicity), m = l1 and
    S = sum exp(l - m): pmax = 1 / S and margin = (exp(l1 - m) - exp(l2 - m)) / S, the
    top-1 minus the top-2 probability.  Commit window positions left to right while
    margin >= tau, stop at the first below, at least one; tau >= 1 commits exactly one.
    """
    x = np.asarray(logits, dtype=np.float64)
    tokens, pmax = accept_rows(x)
    srt = np.sort(x, axis=-1)
    l1 = srt[..., -1]
    l2 = srt[..., -2] if x.shape[-1] > 1 else np.full_like(l1, -np.inf)   # one entry: no top-2
    S = 1.0 / pmax
    margin = (1.0 - np.exp(l2 - l1)) / S
    b, W = margin.shape
    n = np.zeros(b, dtype=np.int32)
    for bi in range(b):
        run = 0
        if tau < 1.0:
            while run < W and margin[bi, run] >= tau:
                run += 1
        n[bi] = max(1, run)
    return tokens, pmax, margin, n


def accept_margin_scalar(logits, tau):
    """Loop form of :func:`accept_margin` (tiny vocabularies): one pass keeping the two
    largest entries, compensated summation for S."""
    x = np.asarray(logits, dtype=np.float64)
    b, W, V = x.shape
    tokens = np.zeros((b, W), dtype=np.int32)
    margin = np.zeros((b, W))
    n = np.zeros(b, dtype=np.int32)
    for bi in range(b):
        for i in range(W):
            row = [float(t) for t in x[bi, i]]
            best, arg, second = row[0], 0, -math.inf
            for vi in range(1, V):
                t = row[vi]
                if t > best:
                    best, second, arg = t, best, vi
                elif t > second:
                    second = t
            tokens[bi, i] = arg
            S = math.fsum(math.exp(t - best) for t in row)
            margin[bi, i] = (1.0 - (math.exp(second - best) if V > 1 else 0.0)) / S
        cnt = 0
        if tau < 1.0:
            for i in range(W):
                if margin[bi, i] >= tau:
                    cnt += 1
                else:
                    break
        n[bi] = max(1, cnt)
    return tokens, margin, n


# ---------------------------------------------------------------------------
# KV commit and cursor advance ([BLOG] "Batching is where methods like this usually die")
# ---------------------------------------------------------------------------

def kv_commit(k_cache, v_cache, cache_len, k_win, v_win, n_accept, batch_min=False):
    """Append accepted window K/V to per-sequence caches and advance the cursors.

    k_cache, v_cache [b, Hkv, cap, D]; cache_len [b]; k_win, v_win [b, W, Hkv, D];
    n_accept [b] in [1, W].  n_b = n_accept[b] (per-sample cursors), or min_b n_accept
    for every sequence (the block-level cache advancing at the batch minimum).  If
    cache_len[b] + n_b > cap nothing is committed for b.  Returns (k_cache', v_cache',
    cache_len', valid [b] bitmask of committed window rows, overflow [b] bool).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    ln = np.array(cache_len, dtype=np.int64, copy=True)
    b, Hkv, cap, D = kc.shape
    W = k_win.shape[1]
    n_acc = np.asarray(n_accept, dtype=np.int64)
    nmin = int(n_acc.min()) if b else 0
    valid = np.zeros(b, dtype=np.uint64)
    over = np.zeros(b, dtype=bool)
    for bi in range(b):
        n = nmin if batch_min else int(n_acc[bi])
        n = max(0, min(n, W))
        start = int(ln[bi])
        if start + n > cap:
            over[bi] = True
            continue
        for i in range(n):
            for g in range(Hkv):
                kc[bi, g, start + i, :] = k_win[bi, i, g, :]
                vc[bi, g, start + i, :] = v_win[bi, i, g, :]
            valid[bi] |= np.uint64(1) << np.uint64(i)
        ln[bi] = start + n
    return kc, vc, ln.astype(np.int32), valid, over


# ---------------------------------------------------------------------------
# Right-shifted cross-entropy L = L_mask + L_AR ([MARS] §3.2 Eq. 3, §3.3 Eq. 4-5)
# ---------------------------------------------------------------------------

def shifted_ce_targets(P, L, B):
    """Per logits row of [prompt; x; x~] (N = P + 2L rows): (target response offset or -1,
    AR weight, mask weight).  Right-shifted logits: row p predicts the token at p + 1.

    * clean row P - 1 + t (t = 0..L-1, row >= 0) predicts x_t: AR weight 1; mask weight 1
      when t is the first offset of a block (t % B == 0), whose context is fully clean;
    * noisy row P + L + j (j = 0..L-2) predicts x_{j+1} when j+1 is not a block start:
      mask weight 1 (context: the clean prefix of earlier blocks plus the masks up to j);
    * every other row predicts nothing.
    """
    N = P + 2 * L
    tgt = np.full(N, -1, dtype=np.int64)
    war = np.zeros(N)
    wmask = np.zeros(N)
    for t in range(L):
        r = P - 1 + t
        if r >= 0:
            tgt[r] = t
            war[r] = 1.0
            if t % B == 0:
                wmask[r] = 1.0
    for j in range(L - 1):
        if (j + 1) % B != 0:
            r = P + L + j
            tgt[r] = j + 1
            wmask[r] = 1.0
    return tgt, war, wmask


def shifted_ce(logits, x, P, L, B):
    """L_mask and L_AR of one batch of logits [b, N, V] for response tokens x [b, L].

    Returns (loss_mask [b], loss_ar [b], dlogits [b, N, V]) in float64, where dlogits is
    the gradient of L_mask + L_AR: (w_ar + w_mask) * (softmax(row) - onehot(target)) on rows
    with a target, zero elsewhere.
    """
    z = np.asarray(logits, dtype=np.float64)
    b, N, V = z.shape
    assert N == P + 2 * L and x.shape == (b, L)
    tgt, war, wmask = shifted_ce_targets(P, L, B)
    rows = np.nonzero(tgt >= 0)[0]
    m = z[:, rows].max(axis=-1, keepdims=True)
    lse = m[..., 0] + np.log(np.exp(z[:, rows] - m).sum(axis=-1))           # [b, R]
    tok = np.asarray(x)[:, tgt[rows]]                                          # [b, R]
    picked = np.take_along_axis(z[:, rows], tok[..., None], axis=-1)[..., 0]
    ce = lse - picked
    loss_ar = (ce * war[rows]).sum(axis=1)
    loss_mask = (ce * wmask[rows]).sum(axis=1)
    d = np.zeros_like(z)
    sm = np.exp(z[:, rows] - lse[..., None])
    for k, r in enumerate(rows):
        g = sm[:, k].copy()
        g[np.arange(b), tok[:, k]] -= 1.0
        d[:, r] = (war[r] + wmask[r]) * g
    return loss_mask, loss_ar, d
