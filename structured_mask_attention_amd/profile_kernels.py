"""Run libmars kernels in isolation for profiler passes (e.g. ``rocprofv3 --pmc ...``).

Usage: python -m structured_mask_attention_amd.profile_kernels [what ...] [--reps N]
  what: attn05 (Qwen2.5-0.5B-shaped training layout), attn7 (7B-shaped), attnlong (long
        7B-shaped), decode (7B-shaped decode step), accept (152k-vocabulary accept),
        bwd05, bwd7, bwdlong (training backward on those layouts), loss05 (training loss with its gradient
        on the 0.5B layout's logits [8, 1280, 151936]), copy (a plain 256 MiB
        device-to-device copy: the calibration of byte counters).
Inputs are the seeded synthetic workloads of ``inputs``; every launch reads fresh copies
in rotation so caches do not hold them between launches of the same kernel.
"""
from __future__ import annotations

import argparse

import torch

from . import inputs as I
from . import (mars_accept, mars_accept_workspace_bytes, mars_attn_bwd, mars_attn_fwd, mars_decode_step,
               mars_decode_workspace_bytes, mars_shifted_ce)

TRAIN = {"attn05": I.QWEN05B, "attn7": I.QWEN7B, "attnlong": I.LONG7B}
BWD = {"bwd05": I.QWEN05B, "bwd7": I.QWEN7B, "bwdlong": I.LONG7B}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("what", nargs="*", default=["attn05", "decode", "accept"])
    ap.add_argument("--reps", type=int, default=6)
    ap.add_argument("--copies", type=int, default=3)
    a = ap.parse_args()
    dev = torch.device("cuda:0")
    for w in a.what:
        if w in TRAIN:
            s = TRAIN[w]
            host = I.train_inputs(s)
            sets = [tuple(t.to(dev) for t in host) for _ in range(a.copies)]
            o = torch.empty_like(sets[0][0])
            for r in range(a.reps):
                mars_attn_fwd(*sets[r % a.copies], s.P, s.L, s.B, out=o)
        elif w in ("decode", "accept"):
            s = I.DECODE7B
            x = I.decode_inputs(s)
            host = (x.q_win, x.k_win, x.v_win, x.k_cache, x.v_cache, x.cache_len, x.logits)
            sets = [tuple(t.to(dev) for t in host) for _ in range(a.copies)]
            if w == "decode":
                ws = torch.empty(mars_decode_workspace_bytes(s.batch, s.hq, s.hkv, s.d, s.W, s.cap),
                                 dtype=torch.uint8, device=dev)
                for r in range(a.reps):
                    mars_decode_step(*sets[r % a.copies][:6], ws=ws)
            else:
                ws = torch.empty(mars_accept_workspace_bytes(s.batch, s.W, s.vocab), dtype=torch.uint8, device=dev)
                for r in range(a.reps):
                    mars_accept(sets[r % a.copies][6], s.tau, ws=ws)
        elif w in BWD:
            s = BWD[w]
            host = I.train_inputs(s)
            sets = [tuple(t.to(dev) for t in host) for _ in range(a.copies)]
            do = I.grad_output(s).to(dev)
            fw = []
            for q, k, v in sets:
                lse = torch.empty((s.batch, s.hq, s.N), dtype=torch.float32, device=dev)
                fw.append((mars_attn_fwd(q, k, v, s.P, s.L, s.B, lse=lse), lse))
            for r in range(a.reps):
                q, k, v = sets[r % a.copies]
                o, lse = fw[r % a.copies]
                mars_attn_bwd(q, k, v, o, lse, do, s.P, s.L, s.B)
        elif w == "loss05":
            s = I.QWEN05B
            logits, tokens = I.ce_inputs(s.batch, s.P, s.L, 151936, 2002, device=dev)
            dl = torch.empty_like(logits)
            for r in range(a.reps):
                mars_shifted_ce(logits, tokens, s.P, s.L, s.B, grad=True, dlogits=dl)
        elif w == "copy":
            n = 256 << 20
            src = [torch.ones(n, dtype=torch.uint8, device=dev) for _ in range(a.copies)]
            dst = torch.empty(n, dtype=torch.uint8, device=dev)
            for r in range(a.reps):
                dst.copy_(src[r % a.copies])
        else:
            raise SystemExit(f"unknown kernel set {w!r}")
        torch.cuda.synchronize()
        print(f"done {w}", flush=True)


if __name__ == "__main__":
    main()
