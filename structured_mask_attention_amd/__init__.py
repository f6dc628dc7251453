"""MARS structured-mask attention on MI355X: Python binding of libmars (include/mars.h).

Same names as the C ABI.  Tensors are torch CUDA (ROCm) tensors used for device memory
and streams only; every step of the computation runs in libmars's HIP kernels.  Calls
are asynchronous on the current stream of the tensors' device.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L

__all__ = [
    "MarsError",
    "mars_abi_version",
    "mars_strerror",
    "mars_attn_fwd",
    "mars_attn_work",
    "mars_attn_bwd_plan",
    "mars_mask_materialize",
    "mars_tile_map",
    "mars_attn_tilelog_geometry",
    "mars_attn_fwd_tilelog",
    "mars_attn_bwd_workspace_bytes",
    "mars_attn_bwd",
    "mars_decode_workspace_bytes",
    "mars_decode_step",
    "mars_decode_step_noalloc",
    "mars_decode_scratch_bytes",
    "mars_accept_workspace_bytes",
    "mars_accept",
    "mars_accept_margin",
    "mars_kv_commit",
    "mars_shifted_ce",
]


class MarsError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = L.load().mars_strerror(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")


def _check(status: int, where: str):
    if status != L.MARS_OK:
        raise MarsError(status, where)


def _ptr(t):
    # ctypes turns a Python int into the void* argument itself.
    return None if t is None else t.data_ptr()


def _spec_check(t, name, dtype, shape=None, contiguous=False):
    """dtype (TypeError), shape and contiguity (ValueError) of one tensor argument."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    dts = dtype if isinstance(dtype, tuple) else (dtype,)
    if t.dtype not in dts:
        raise TypeError(f"{name} must have dtype {' or '.join(str(d) for d in dts)}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _validate(specs):
    """Check every tensor argument before anything reaches the C ABI: first each one's dtype,
    shape and contiguity, then that all of them live on one device (ROCm) - the device of the
    first.  The library reads every buffer with the element type and layout its descriptor
    states, so a wrong dtype or a host pointer must never get that far.
    specs: (tensor or None, name, dtype(s), shape or None, contiguous) tuples; None skipped."""
    specs = [sp for sp in specs if sp[0] is not None]
    for t, name, dtype, shape, contiguous in specs:
        _spec_check(t, name, dtype, shape, contiguous)
    dev = None
    for t, name, *_ in specs:
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a device (ROCm) tensor, got one on {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other arguments on {dev}")


def _out(t, shape, dtype, dev):
    """An output the kernels write densely: the caller's (validated) tensor, or a new one."""
    return torch.empty(shape, dtype=dtype, device=dev) if t is None else t


# The raw handle of a device's current stream, without building a torch Stream object per
# call (the binding's host time per call bounds back-to-back launches of short kernels).
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t):
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


_DESCS = {}


def _memo(key, build):
    """Descriptors depend only on shapes, strides and scalars: build each one once (the
    C side copies nothing from them after the call returns, so sharing is safe)."""
    d = _DESCS.get(key)
    if d is None:
        if len(_DESCS) > 512:
            _DESCS.clear()
        d = _DESCS[key] = build()
    return d


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return L.MARS_DTYPE_BF16
    if dt == torch.float32:
        return L.MARS_DTYPE_FP32
    raise TypeError(f"unsupported dtype {dt}")


def _s3(t, dims=(0, 1, 2)):
    if t.numel() == 0:   # no element is ever addressed: report dense strides
        dense = [1] * t.dim()
        for i in range(t.dim() - 2, -1, -1):
            dense[i] = dense[i + 1] * max(t.shape[i + 1], 1)
        return L.I64x3(*(dense[i] for i in dims))
    if t.stride(-1) != 1:
        raise ValueError("innermost dimension must be contiguous")
    return L.I64x3(*(t.stride(i) for i in dims))


def mars_abi_version() -> int:
    return L.load().mars_abi_version()


def mars_strerror(status: int) -> str:
    return L.load().mars_strerror(status).decode()


def attn_desc(batch, hq, hkv, d, P, Lr, B, dtype=torch.bfloat16, scale=0.0, q=None, k=None, v=None, o=None):
    desc = L.AttnDesc()
    desc.batch, desc.n_q_heads, desc.n_kv_heads, desc.head_dim = batch, hq, hkv, d
    desc.prompt_len, desc.resp_len, desc.block = P, Lr, B
    desc.dtype = _dtype_code(dtype)
    desc.scale = float(scale)
    desc.reserved = 0
    N = P + 2 * Lr
    dense_q = (N * hq * d, hq * d, d)
    dense_kv = (N * hkv * d, hkv * d, d)
    desc.q_strides = _s3(q) if q is not None else L.I64x3(*dense_q)
    desc.k_strides = _s3(k) if k is not None else L.I64x3(*dense_kv)
    desc.v_strides = _s3(v) if v is not None else L.I64x3(*dense_kv)
    desc.o_strides = _s3(o) if o is not None else L.I64x3(*dense_q)
    return desc


def _attn_specs(q, k, v, o, P, Lr, dtypes=(torch.bfloat16, torch.float32), lse=None, lse_required=False):
    """Argument specs of the training-layout calls (shapes from q and k)."""
    _spec_check(q, "q", dtypes)
    _spec_check(k, "k", q.dtype)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [batch, N, n_q_heads, head_dim] and k [batch, N, n_kv_heads, head_dim]")
    b, N, hq, d = q.shape
    hkv = k.shape[2]
    if N != P + 2 * Lr:
        raise ValueError(f"sequence length {N} != P + 2L = {P + 2 * Lr}")
    if lse_required and lse is None:
        raise ValueError("lse (the forward's fp32 [b, Hq, N] log-sum-exp) is required")
    return [(q, "q", q.dtype, None, False), (k, "k", q.dtype, (b, N, hkv, d), False),
            (v, "v", q.dtype, (b, N, hkv, d), False), (o, "out", q.dtype, q.shape, False),
            (lse, "lse", torch.float32, (b, hq, N), True)]


def _attn_desc_from(q, k, v, o, P, Lr, B, scale):
    b, N, hq, d = q.shape
    return attn_desc(b, hq, k.shape[2], d, P, Lr, B, q.dtype, scale, q, k, v, o)


def mars_attn_fwd(q, k, v, prompt_len, resp_len, block, scale=0.0, out=None, lse=None):
    """O = softmax(scale Q K^T + M) V over [prompt; x; x~]; q [b,N,Hq,D], k/v [b,N,Hkv,D].

    ``lse``: optional fp32 [b, Hq, N] tensor to receive the log-sum-exp.  Returns ``out``.
    """
    _validate(_attn_specs(q, k, v, out, prompt_len, resp_len, lse=lse))
    out = torch.empty_like(q) if out is None else out
    desc = _attn_desc_from(q, k, v, out, prompt_len, resp_len, block, scale)
    _check(L.load().mars_attn_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                  _stream(q)), "mars_attn_fwd")
    return out


def mars_attn_bwd_workspace_bytes(batch, hq, hkv, d, P, Lr, B, dtype=torch.bfloat16):
    """Workspace bytes of :func:`mars_attn_bwd` (see mars.h)."""
    desc = attn_desc(batch, hq, hkv, d, P, Lr, B, dtype)
    n = ctypes.c_size_t()
    _check(L.load().mars_attn_bwd_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
           "mars_attn_bwd_workspace_bytes")
    return n.value


def mars_attn_bwd_plan(batch, hq, hkv, d, P, Lr, B):
    """The dK/dV schedule of :func:`mars_attn_bwd` for a layout (host only, see mars.h):
    dict with chunk_tiles, max_chunks, items and work_list."""
    desc = attn_desc(batch, hq, hkv, d, P, Lr, B, torch.bfloat16)
    tc, nch, wl = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    n = ctypes.c_int64()
    _check(L.load().mars_attn_bwd_plan(ctypes.byref(desc), ctypes.byref(tc), ctypes.byref(nch), ctypes.byref(n),
                                       ctypes.byref(wl)), "mars_attn_bwd_plan")
    return {"chunk_tiles": tc.value, "max_chunks": nch.value, "items": n.value, "work_list": bool(wl.value)}


def mars_attn_bwd(q, k, v, o, lse, dout, prompt_len, resp_len, block, scale=0.0, dq=None, dk=None, dv=None,
                  ws=None):
    """Gradients (dq, dk, dv) of mars_attn_fwd for the upstream gradient ``dout``.

    q/k/v: the forward's inputs; o, lse: its outputs (lse fp32 [b, Hq, N]); dout like o.
    ``ws``: optional uint8 device tensor of at least mars_attn_bwd_workspace_bytes.
    """
    specs = _attn_specs(q, k, v, o, prompt_len, resp_len, torch.bfloat16, lse=lse, lse_required=True)
    specs[3] = (o, "o", torch.bfloat16, q.shape, False)
    specs += [(dout, "dout", torch.bfloat16, q.shape, False), (dq, "dq", torch.bfloat16, q.shape, False),
              (dk, "dk", torch.bfloat16, k.shape, False), (dv, "dv", torch.bfloat16, k.shape, False),
              (ws, "ws", torch.uint8, None, False)]
    _validate(specs)
    desc = _attn_desc_from(q, k, v, o, prompt_len, resp_len, block, scale)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    gs = L.AttnBwdStrides()
    gs.do_strides, gs.dq_strides, gs.dk_strides, gs.dv_strides = _s3(dout), _s3(dq), _s3(dk), _s3(dv)
    n = ctypes.c_size_t()
    _check(L.load().mars_attn_bwd_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "mars_attn_bwd_workspace_bytes")
    ws = torch.empty(max(n.value, 16), dtype=torch.uint8, device=q.device) if ws is None else ws
    _check(L.load().mars_attn_bwd(ctypes.byref(desc), ctypes.byref(gs), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                  _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ctypes.c_size_t(ws.numel()),
                                  _stream(q)), "mars_attn_bwd")
    return dq, dk, dv


def mars_attn_work(batch, hq, hkv, d, P, Lr, B, bm=128, bn=128, dtype=torch.bfloat16):
    """(nnz, visible_elems) per (batch, head), host-side (see mars.h)."""
    desc = attn_desc(batch, hq, hkv, d, P, Lr, B, dtype)
    nnz, vis = ctypes.c_int64(), ctypes.c_int64()
    _check(L.load().mars_attn_work(ctypes.byref(desc), bm, bn, ctypes.byref(nnz), ctypes.byref(vis)),
           "mars_attn_work")
    return nnz.value, vis.value


def mars_mask_materialize(P, Lr, B, device="cuda"):
    N = P + 2 * Lr
    mask = torch.empty((N, N), dtype=torch.uint8, device=device)
    desc = attn_desc(1, 1, 1, 64, P, Lr, B)
    _check(L.load().mars_mask_materialize(ctypes.byref(desc), _ptr(mask), _stream(mask)), "mars_mask_materialize")
    return mask


def mars_tile_map(P, Lr, B, bm, bn, device="cuda"):
    N = P + 2 * Lr
    m = torch.empty(((N + bm - 1) // bm, (N + bn - 1) // bn), dtype=torch.int8, device=device)
    desc = attn_desc(1, 1, 1, 64, P, Lr, B)
    _check(L.load().mars_tile_map(ctypes.byref(desc), bm, bn, _ptr(m), _stream(m)), "mars_tile_map")
    return m


def mars_attn_tilelog_geometry(batch, hq, hkv, d, P, Lr, B):
    desc = attn_desc(batch, hq, hkv, d, P, Lr, B)
    rb, kb, rows = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check(L.load().mars_attn_tilelog_geometry(ctypes.byref(desc), ctypes.byref(rb), ctypes.byref(kb),
                                               ctypes.byref(rows)), "mars_attn_tilelog_geometry")
    return rb.value, kb.value, rows.value


def mars_attn_fwd_tilelog(q, k, v, prompt_len, resp_len, block, scale=0.0, out=None, lse=None):
    """bf16 forward that also returns the kernel's tile log int8 [b, Hkv, row groups, key groups]."""
    _validate(_attn_specs(q, k, v, out, prompt_len, resp_len, torch.bfloat16, lse=lse))
    out = torch.empty_like(q) if out is None else out
    desc = _attn_desc_from(q, k, v, out, prompt_len, resp_len, block, scale)
    rb, kb, rows = mars_attn_tilelog_geometry(q.shape[0], q.shape[2], k.shape[2], q.shape[3],
                                              prompt_len, resp_len, block)
    N = q.shape[1]
    log = torch.zeros((q.shape[0], k.shape[2], (rows + rb - 1) // rb, (N + kb - 1) // kb),
                      dtype=torch.int8, device=q.device)
    _check(L.load().mars_attn_fwd_tilelog(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                          _ptr(log), _stream(q)), "mars_attn_fwd_tilelog")
    return out, log


def decode_desc(batch, hq, hkv, d, W, cap, scale=0.0, qw=None, kw=None, vw=None, kc=None, vc=None, o=None):
    desc = L.DecodeDesc()
    desc.batch, desc.n_q_heads, desc.n_kv_heads, desc.head_dim = batch, hq, hkv, d
    desc.window, desc.cache_capacity = W, cap
    desc.dtype = L.MARS_DTYPE_BF16
    desc.scale = float(scale)
    desc.qw_strides = _s3(qw) if qw is not None else L.I64x3(W * hq * d, hq * d, d)
    desc.kw_strides = _s3(kw) if kw is not None else L.I64x3(W * hkv * d, hkv * d, d)
    desc.vw_strides = _s3(vw) if vw is not None else L.I64x3(W * hkv * d, hkv * d, d)
    desc.kc_strides = _s3(kc) if kc is not None else L.I64x3(hkv * cap * d, cap * d, d)
    desc.vc_strides = _s3(vc) if vc is not None else L.I64x3(hkv * cap * d, cap * d, d)
    desc.o_strides = _s3(o) if o is not None else L.I64x3(W * hq * d, hq * d, d)
    return desc


def mars_decode_workspace_bytes(batch, hq, hkv, d, W, cap):
    desc = decode_desc(batch, hq, hkv, d, W, cap)
    n = ctypes.c_size_t()
    _check(L.load().mars_decode_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "mars_decode_workspace_bytes")
    return n.value


def mars_decode_step(q_win, k_win, v_win, k_cache, v_cache, cache_len, scale=0.0, out=None, ws=None):
    """Window rows [b,W,Hq,D] attend to cache [b,Hkv,cap,D] prefix of cache_len[b] plus the causal window."""
    _spec_check(q_win, "q_win", torch.bfloat16)
    _spec_check(k_cache, "k_cache", torch.bfloat16)
    if q_win.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q_win must be [batch, W, n_q_heads, D] and k_cache [batch, n_kv_heads, cap, D]")
    b, W, hq, d = q_win.shape
    hkv, cap = k_cache.shape[1], k_cache.shape[2]
    _validate([(q_win, "q_win", torch.bfloat16, None, False),
               (k_win, "k_win", torch.bfloat16, (b, W, hkv, d), False),
               (v_win, "v_win", torch.bfloat16, (b, W, hkv, d), False),
               (k_cache, "k_cache", torch.bfloat16, (b, hkv, cap, d), False),
               (v_cache, "v_cache", torch.bfloat16, (b, hkv, cap, d), False),
               (cache_len, "cache_len", torch.int32, (b,), True),
               (out, "out", torch.bfloat16, q_win.shape, False),
               (ws, "ws", torch.uint8, None, False)])
    out = torch.empty_like(q_win) if out is None else out
    key = ("dec", b, hq, hkv, d, W, cap, float(scale), q_win.stride(), k_win.stride(), v_win.stride(),
           k_cache.stride(), v_cache.stride(), out.stride())
    desc = _memo(key, lambda: decode_desc(b, hq, hkv, d, W, cap, scale, q_win, k_win, v_win, k_cache, v_cache, out))
    if ws is None:
        ws = torch.empty(max(mars_decode_workspace_bytes(b, hq, hkv, d, W, cap), 16), dtype=torch.uint8,
                         device=q_win.device)
    _check(L.load().mars_decode_step(ctypes.byref(desc), _ptr(q_win), _ptr(k_win), _ptr(v_win), _ptr(k_cache),
                                     _ptr(v_cache), _ptr(cache_len), _ptr(out), _ptr(ws), ws.numel(),
                                     _stream(q_win)), "mars_decode_step")
    return out


def mars_decode_scratch_bytes():
    """Size of the per-device scratch array of :func:`mars_decode_step_noalloc`."""
    n = ctypes.c_size_t()
    _check(L.load().mars_decode_scratch_bytes(ctypes.byref(n)), "mars_decode_scratch_bytes")
    return n.value


def mars_decode_step_noalloc(q_win, k_win, v_win, k_cache, v_cache, cache_len, scale=0.0, out=None):
    """:func:`mars_decode_step` without a workspace: the library keeps the chunk partials in
    its own per-device scratch array (for callers that cannot allocate).  ``out`` must be
    given when the caller cannot allocate either (otherwise one is made here)."""
    _spec_check(q_win, "q_win", torch.bfloat16)
    _spec_check(k_cache, "k_cache", torch.bfloat16)
    if q_win.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q_win must be [batch, W, n_q_heads, D] and k_cache [batch, n_kv_heads, cap, D]")
    b, W, hq, d = q_win.shape
    hkv, cap = k_cache.shape[1], k_cache.shape[2]
    _validate([(q_win, "q_win", torch.bfloat16, None, False),
               (k_win, "k_win", torch.bfloat16, (b, W, hkv, d), False),
               (v_win, "v_win", torch.bfloat16, (b, W, hkv, d), False),
               (k_cache, "k_cache", torch.bfloat16, (b, hkv, cap, d), False),
               (v_cache, "v_cache", torch.bfloat16, (b, hkv, cap, d), False),
               (cache_len, "cache_len", torch.int32, (b,), True),
               (out, "out", torch.bfloat16, q_win.shape, False)])
    out = torch.empty_like(q_win) if out is None else out
    key = ("dec", b, hq, hkv, d, W, cap, float(scale), q_win.stride(), k_win.stride(), v_win.stride(),
           k_cache.stride(), v_cache.stride(), out.stride())
    desc = _memo(key, lambda: decode_desc(b, hq, hkv, d, W, cap, scale, q_win, k_win, v_win, k_cache, v_cache, out))
    _check(L.load().mars_decode_step_noalloc(ctypes.byref(desc), _ptr(q_win), _ptr(k_win), _ptr(v_win),
                                             _ptr(k_cache), _ptr(v_cache), _ptr(cache_len), _ptr(out),
                                             _stream(q_win)), "mars_decode_step_noalloc")
    return out


def accept_desc(batch, W, V, tau, batch_stride=None, row_stride=None):
    desc = L.AcceptDesc()
    desc.batch, desc.window, desc.vocab = batch, W, V
    desc.dtype = L.MARS_DTYPE_BF16
    desc.batch_stride = W * V if batch_stride is None else batch_stride
    desc.row_stride = V if row_stride is None else row_stride
    desc.tau = float(tau)
    desc.min_accept = 1
    return desc


def mars_accept_workspace_bytes(batch, W, V, tau=0.95):
    desc = accept_desc(batch, W, V, tau)
    n = ctypes.c_size_t()
    _check(L.load().mars_accept_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "mars_accept_workspace_bytes")
    return n.value


def mars_accept(logits, tau, ws=None, tokens=None, pmax=None, n_accept=None):
    """logits bf16 [b, W, V] -> (tokens int32 [b,W], pmax fp32 [b,W], n_accept int32 [b]).

    ``ws``: optional device workspace (uint8, at least mars_accept_workspace_bytes).
    """
    _spec_check(logits, "logits", torch.bfloat16)
    if logits.dim() != 3:
        raise ValueError("logits must be [batch, W, vocab]")
    b, W, V = logits.shape
    _validate([(logits, "logits", torch.bfloat16, None, False), (tokens, "tokens", torch.int32, (b, W), True),
               (pmax, "pmax", torch.float32, (b, W), True), (n_accept, "n_accept", torch.int32, (b,), True),
               (ws, "ws", torch.uint8, None, False)])
    if logits.stride(-1) != 1:
        raise ValueError("vocab dimension must be contiguous")
    desc = _memo(("acc", b, W, V, float(tau), logits.stride(0), logits.stride(1)),
                 lambda: accept_desc(b, W, V, tau, logits.stride(0), logits.stride(1)))
    dev = logits.device
    tokens = _out(tokens, (b, W), torch.int32, dev)
    pmax = _out(pmax, (b, W), torch.float32, dev)
    n_accept = _out(n_accept, (b,), torch.int32, dev)
    if ws is None:
        ws = torch.empty(max(mars_accept_workspace_bytes(b, W, V, tau), 16), dtype=torch.uint8, device=dev)
    _check(L.load().mars_accept(ctypes.byref(desc), _ptr(logits), _ptr(tokens), _ptr(pmax), _ptr(n_accept),
                                _ptr(ws), ws.numel(), _stream(logits)), "mars_accept")
    return tokens, pmax, n_accept


def mars_accept_margin(logits, tau, ws=None, tokens=None, pmax=None, margin=None, n_accept=None):
    """Margin gate: logits bf16 [b, W, V] -> (tokens, pmax, margin fp32 [b,W], n_accept [b]).

    margin = top-1 minus top-2 probability; n_accept = leading run with margin >= tau, at
    least one.  ``ws``: optional device workspace (uint8, at least mars_accept_workspace_bytes).
    """
    _spec_check(logits, "logits", torch.bfloat16)
    if logits.dim() != 3:
        raise ValueError("logits must be [batch, W, vocab]")
    b, W, V = logits.shape
    _validate([(logits, "logits", torch.bfloat16, None, False), (tokens, "tokens", torch.int32, (b, W), True),
               (pmax, "pmax", torch.float32, (b, W), True), (margin, "margin", torch.float32, (b, W), True),
               (n_accept, "n_accept", torch.int32, (b,), True), (ws, "ws", torch.uint8, None, False)])
    if logits.stride(-1) != 1:
        raise ValueError("vocab dimension must be contiguous")
    desc = _memo(("acc", b, W, V, float(tau), logits.stride(0), logits.stride(1)),
                 lambda: accept_desc(b, W, V, tau, logits.stride(0), logits.stride(1)))
    dev = logits.device
    tokens = _out(tokens, (b, W), torch.int32, dev)
    pmax = _out(pmax, (b, W), torch.float32, dev)
    margin = _out(margin, (b, W), torch.float32, dev)
    n_accept = _out(n_accept, (b,), torch.int32, dev)
    if ws is None:
        ws = torch.empty(max(mars_accept_workspace_bytes(b, W, V, tau), 16), dtype=torch.uint8, device=dev)
    _check(L.load().mars_accept_margin(ctypes.byref(desc), _ptr(logits), _ptr(tokens), _ptr(pmax), _ptr(margin),
                                       _ptr(n_accept), _ptr(ws), ws.numel(), _stream(logits)), "mars_accept_margin")
    return tokens, pmax, margin, n_accept


def mars_kv_commit(k_win, v_win, n_accept, k_cache, v_cache, cache_len, batch_min=False, valid=None, overflow=None):
    """Append accepted window K/V ([b, W, Hkv, D]) to the caches ([b, Hkv, cap, D]) at the
    cursors ``cache_len`` (int32 [b], updated in place) and advance them by n_accept[b]
    (or the batch minimum).  Returns (valid uint64-as-int64 [b], overflow int32 [b])."""
    _spec_check(k_win, "k_win", torch.bfloat16)
    _spec_check(k_cache, "k_cache", torch.bfloat16)
    if k_win.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("k_win must be [batch, W, n_kv_heads, D] and k_cache [batch, n_kv_heads, cap, D]")
    b, W, hkv, d = k_win.shape
    cap = k_cache.shape[2]
    _validate([(k_win, "k_win", torch.bfloat16, None, False),
               (v_win, "v_win", torch.bfloat16, (b, W, hkv, d), False),
               (n_accept, "n_accept", torch.int32, (b,), True),
               (k_cache, "k_cache", torch.bfloat16, (b, hkv, cap, d), False),
               (v_cache, "v_cache", torch.bfloat16, (b, hkv, cap, d), False),
               (cache_len, "cache_len", torch.int32, (b,), True),
               (valid, "valid", torch.int64, (b,), True), (overflow, "overflow", torch.int32, (b,), True)])
    key = ("commit", b, hkv, d, W, cap, k_win.stride(), v_win.stride(), k_cache.stride(), v_cache.stride())
    desc = _memo(key, lambda: decode_desc(b, hkv, hkv, d, W, cap, 0.0, None, k_win, v_win, k_cache, v_cache, None))
    dev = k_win.device
    valid = _out(valid, (b,), torch.int64, dev)
    overflow = _out(overflow, (b,), torch.int32, dev)
    policy = L.MARS_COMMIT_BATCH_MIN if batch_min else L.MARS_COMMIT_PER_SAMPLE
    _check(L.load().mars_kv_commit(ctypes.byref(desc), _ptr(k_win), _ptr(v_win), _ptr(n_accept), _ptr(k_cache),
                                   _ptr(v_cache), _ptr(cache_len), _ptr(valid), _ptr(overflow), policy,
                                   _stream(k_win)), "mars_kv_commit")
    return valid, overflow


def ce_desc(batch, P, Lr, B, V, logits=None, dlogits=None, tokens=None):
    desc = L.CeDesc()
    desc.batch, desc.prompt_len, desc.resp_len, desc.block, desc.vocab = batch, P, Lr, B, V
    desc.dtype = L.MARS_DTYPE_BF16
    N = P + 2 * Lr
    ls = (logits.stride(0), logits.stride(1)) if logits is not None else (N * V, V)
    ds = (dlogits.stride(0), dlogits.stride(1)) if dlogits is not None else (N * V, V)
    desc.logits_strides = (ctypes.c_int64 * 2)(*ls)
    desc.dlogits_strides = (ctypes.c_int64 * 2)(*ds)
    desc.tokens_stride = tokens.stride(0) if tokens is not None else Lr
    return desc


def mars_shifted_ce(logits, tokens, prompt_len, resp_len, block, grad=False, dlogits=None, ws=None):
    """L_mask, L_AR (fp32 [b] each) of logits bf16 [b, N, V] for response tokens int32
    [b, L]; with ``grad`` also dlogits bf16 [b, N, V].  Returns (loss_mask, loss_ar, dlogits)."""
    _spec_check(logits, "logits", torch.bfloat16)
    if logits.dim() != 3:
        raise ValueError("logits must be [batch, N, vocab]")
    b, N, V = logits.shape
    if N != prompt_len + 2 * resp_len:
        raise ValueError(f"logits rows {N} != P + 2L = {prompt_len + 2 * resp_len}")
    _validate([(logits, "logits", torch.bfloat16, None, False), (tokens, "tokens", torch.int32, (b, resp_len), False),
               (dlogits, "dlogits", torch.bfloat16, logits.shape, False), (ws, "ws", torch.uint8, None, False)])
    dev = logits.device
    if logits.stride(-1) != 1 or tokens.stride(-1) != 1 or (dlogits is not None and dlogits.stride(-1) != 1):
        raise ValueError("vocab and token dimensions must be contiguous")
    if grad and dlogits is None:
        dlogits = torch.empty_like(logits)
    desc = ce_desc(b, prompt_len, resp_len, block, V, logits, dlogits, tokens)
    n = ctypes.c_size_t()
    _check(L.load().mars_shifted_ce_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
           "mars_shifted_ce_workspace_bytes")
    ws = torch.empty(max(n.value, 16), dtype=torch.uint8, device=dev) if ws is None else ws
    lm = torch.empty((b,), dtype=torch.float32, device=dev)
    la = torch.empty((b,), dtype=torch.float32, device=dev)
    _check(L.load().mars_shifted_ce(ctypes.byref(desc), _ptr(logits), _ptr(tokens), _ptr(lm), _ptr(la),
                                    _ptr(dlogits), _ptr(ws), ws.numel(), _stream(logits)), "mars_shifted_ce")
    return lm, la, dlogits
