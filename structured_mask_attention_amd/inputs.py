"""Seeded synthetic inputs shaped like the MARS workloads.

This module holds shapes and random draws only, none of the method's arithmetic.
Both the HIP-path tests/bench and the CPU oracle consume what it returns.

Recipe (one NumPy PCG64 generator per workload, seeded):
  * training layout: draw Q, then K, then V as float32 standard normals, multiply by
    the workload's input scale, and round to bfloat16 with round-to-nearest-even
    (torch's CPU cast) unless the workload is float32;
  * decode step: draw the cache lengths (integers uniform on [len_lo, len_hi]), then
    window Q, K, V, then the K and V caches (full capacity), then the logits
    (standard normal), the spike heights (uniform on [0, 20)) and the spike token
    ids (uniform on [0, V)); the spike is added in float32 before the bf16 rounding.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class TrainShape:
    name: str
    batch: int
    hq: int
    hkv: int
    d: int
    P: int
    L: int
    B: int
    dtype: str          # "bf16" or "fp32"
    in_scale: float
    seed: int

    @property
    def N(self) -> int:
        return self.P + 2 * self.L


@dataclass(frozen=True)
class DecodeShape:
    name: str
    batch: int
    hq: int
    hkv: int
    d: int
    W: int
    cap: int
    len_lo: int
    len_hi: int
    vocab: int
    tau: float
    in_scale: float
    seed: int
    spike_hi: float = 20.0


# The five workloads: a tiny fp32 case, Qwen2.5-0.5B- and 7B-shaped training layouts,
# a 7B-shaped decode step with a 152k vocabulary, and a long 7B-shaped layout.
TINY = TrainShape("tiny_fp32_P16_L64_B4", 1, 1, 1, 64, 16, 64, 4, "fp32", 1.0, 1001)
QWEN05B = TrainShape("qwen2.5-0.5b_train_b8_P256_L512_B4", 8, 14, 2, 64, 256, 512, 4, "bf16", 0.5, 1002)
QWEN7B = TrainShape("qwen2.5-7b_train_b4_P512_L1536_B8", 4, 28, 4, 128, 512, 1536, 8, "bf16", 0.5, 1003)
DECODE7B = DecodeShape("qwen2.5-7b_decode_b32_W4_len512-4096_V152064", 32, 28, 4, 128, 4, 4096,
                       512, 4096, 152064, 0.95, 0.5, 1004)
LONG7B = TrainShape("long_7b_train_b1_P1024_L7168_B32", 1, 28, 4, 128, 1024, 7168, 32, "bf16", 0.5, 1005)

TRAIN_SHAPES = {s.name: s for s in (TINY, QWEN05B, QWEN7B, LONG7B)}


def to_bf16(x: np.ndarray) -> torch.Tensor:
    """float32 array -> bfloat16 CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def as_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a (bf16 or fp32) CPU tensor."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def train_inputs(s: TrainShape, seed: int | None = None):
    """Q [b,N,Hq,D], K, V [b,N,Hkv,D] as CPU tensors in the workload's dtype."""
    rng = np.random.default_rng(s.seed if seed is None else seed)
    shapes = [(s.batch, s.N, s.hq, s.d), (s.batch, s.N, s.hkv, s.d), (s.batch, s.N, s.hkv, s.d)]
    out = []
    for shp in shapes:
        x = rng.standard_normal(shp, dtype=np.float32) * np.float32(s.in_scale)
        out.append(to_bf16(x) if s.dtype == "bf16" else torch.from_numpy(x))
    return tuple(out)


def small_train_inputs(batch, hq, hkv, d, P, L, seed, dtype="bf16", in_scale=0.5):
    """Like :func:`train_inputs` for an ad-hoc shape (parity sweeps, edge cases)."""
    s = TrainShape("adhoc", batch, hq, hkv, d, P, L, 1, dtype, in_scale, seed)
    return train_inputs(s)


def grad_output(s: TrainShape, seed: int | None = None, scale: float = 0.5):
    """dL/dO for the backward: [b, N, Hq, D] ~ N(0, 1) * scale in the workload's dtype, drawn
    from its own stream (seed + 7919) so that Q/K/V stay those of :func:`train_inputs`."""
    rng = np.random.default_rng((s.seed if seed is None else seed) + 7919)
    x = rng.standard_normal((s.batch, s.N, s.hq, s.d), dtype=np.float32) * np.float32(scale)
    return to_bf16(x) if s.dtype == "bf16" else torch.from_numpy(x)


def small_grad_output(batch, hq, d, P, L, seed, dtype="bf16", scale=0.5):
    """Like :func:`grad_output` for an ad-hoc shape."""
    s = TrainShape("adhoc", batch, hq, 1, d, P, L, 1, dtype, 0.5, seed)
    return grad_output(s, scale=scale)


@dataclass
class DecodeInputs:
    cache_len: torch.Tensor   # int32 [b]
    q_win: torch.Tensor       # bf16 [b, W, Hq, D]
    k_win: torch.Tensor       # bf16 [b, W, Hkv, D]
    v_win: torch.Tensor
    k_cache: torch.Tensor     # bf16 [b, Hkv, cap, D]
    v_cache: torch.Tensor
    logits: torch.Tensor      # bf16 [b, W, V]
    spike_ids: np.ndarray = field(default=None)
    spike_heights: np.ndarray = field(default=None)


def decode_inputs(s: DecodeShape, seed: int | None = None, with_logits: bool = True) -> DecodeInputs:
    rng = np.random.default_rng(s.seed if seed is None else seed)
    lens = rng.integers(s.len_lo, s.len_hi, size=s.batch, endpoint=True).astype(np.int32)
    sc = np.float32(s.in_scale)
    q = rng.standard_normal((s.batch, s.W, s.hq, s.d), dtype=np.float32) * sc
    kw = rng.standard_normal((s.batch, s.W, s.hkv, s.d), dtype=np.float32) * sc
    vw = rng.standard_normal((s.batch, s.W, s.hkv, s.d), dtype=np.float32) * sc
    kc = rng.standard_normal((s.batch, s.hkv, s.cap, s.d), dtype=np.float32) * sc
    vc = rng.standard_normal((s.batch, s.hkv, s.cap, s.d), dtype=np.float32) * sc
    logits = heights = ids = None
    if with_logits:
        logits = rng.standard_normal((s.batch, s.W, s.vocab), dtype=np.float32)
        heights = rng.uniform(0.0, s.spike_hi, size=(s.batch, s.W)).astype(np.float32)
        ids = rng.integers(0, s.vocab, size=(s.batch, s.W))
        bi, wi = np.meshgrid(np.arange(s.batch), np.arange(s.W), indexing="ij")
        logits[bi, wi, ids] += heights
    return DecodeInputs(
        cache_len=torch.from_numpy(lens),
        q_win=to_bf16(q), k_win=to_bf16(kw), v_win=to_bf16(vw),
        k_cache=to_bf16(kc), v_cache=to_bf16(vc),
        logits=to_bf16(logits) if with_logits else None,
        spike_ids=ids, spike_heights=heights,
    )


def logits_inputs(batch, W, vocab, seed, spike_hi=20.0):
    """Logits only, same recipe as the decode workload (standard normal + one spike per row)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((batch, W, vocab), dtype=np.float32)
    h = rng.uniform(0.0, spike_hi, size=(batch, W)).astype(np.float32)
    ids = rng.integers(0, vocab, size=(batch, W))
    bi, wi = np.meshgrid(np.arange(batch), np.arange(W), indexing="ij")
    x[bi, wi, ids] += h
    return to_bf16(x)


def ce_inputs(batch, P, L, vocab, seed, device="cpu", spike_hi=20.0):
    """Logits bf16 [batch, P + 2L, vocab] and response tokens int32 [batch, L] for the
    training loss.  Drawn with one torch generator on ``device`` (so the full-size
    workload is made on the GPU without a host copy), in this order: logits (float32
    standard normal), one spike per row (height uniform on [0, spike_hi) at a uniform
    token id, added in float32 before the bf16 rounding), then the tokens (uniform on
    [0, vocab))."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    N = P + 2 * L
    x = torch.randn((batch, N, vocab), generator=g, dtype=torch.float32, device=device)
    h = torch.rand((batch, N), generator=g, dtype=torch.float32, device=device) * spike_hi
    ids = torch.randint(0, vocab, (batch, N), generator=g, device=device)
    x.scatter_add_(2, ids[..., None], h[..., None])
    logits = x.to(torch.bfloat16)
    del x
    tokens = torch.randint(0, vocab, (batch, L), generator=g, device=device).to(torch.int32)
    return logits, tokens
