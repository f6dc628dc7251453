#!/usr/bin/env python3
"""Benchmark of the MARS hot path on one MI355X.

One step = one pass of the whole path on synthetic, seeded inputs resident in HBM:
  1. mars_attn_fwd on the Qwen2.5-0.5B-shaped training layout (batch 8, 14/2 heads,
     head_dim 64, P=256, L=512, B=4)                          -> visible-tile TFLOP/s;
  2. mars_decode_step on the Qwen2.5-7B-shaped decode workload (32 sequences, 28/4 heads,
     head_dim 128, cache lengths U[512, 4096], 4 window rows)  -> GB/s;
  3. mars_accept on its logits [32, 4, 152064] at tau = 0.95   -> GB/s (the margin gate,
     mars_accept_margin, is timed beside it and reported in the decode section, and so is
     mars_kv_commit, the loop's cache append and cursor advance);
  decode tokens/s = sum(n_accept) / (t_decode + t_accept)  (one attention layer + accept).
The timed region is exactly K whole steps (HIP events at its ends, on the launch stream);
per-kernel durations come from groups of K back-to-back launches of one kernel (events
around each group, three groups, mean).  Three independent
copies of every input rotate across steps, so a step reads data last touched about 700 MB
earlier and the 256 MB Infinity Cache holds none of it (no dirty flush traffic either).
The 7B-shaped and long training layouts are timed as well (own events) and reported, and so
is the training backward (mars_attn_bwd: dQ, dK, dV) on all three layouts (counted as five
products over the forward's visible tiles), and the training loss (mars_shifted_ce: L_mask +
L_AR with the logits gradient on [8, 1280, 151936] bf16 logits -> GB/s of one read of the
logits and one write of the gradient).
The CPU baseline is the fp64 oracle on a bounded sample of the same workloads.

Prints one JSON line.  Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "visible-tile TFLOP/s (train layout) + decode-step tokens/s at τ=0.95, 1 GPU"
MARGIN_TAU = 0.3              # margin-gate threshold for its timing line (the pages give no value)
QWEN05B_VOCAB = 151936        # Qwen2.5-0.5B output vocabulary (training-loss timing)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-layouts", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the training backward figures")
    ap.add_argument("--no-loss", action="store_true", help="skip the training loss (L_mask + L_AR) figures")
    ap.add_argument("--copies", type=int, default=3, help="rotated input copies (1 = warm caches)")
    return ap.parse_args()


def train_flops(M, s):
    """(FLOP_vt on the fixed 128x128 grid, FLOP_alg from the exact nnz) of one forward."""
    nnz, vis = M.mars_attn_work(s.batch, s.hq, s.hkv, s.d, s.P, s.L, s.B, 128, 128)
    per = 4.0 * s.d * s.batch * s.hq
    return per * vis, per * nnz


def executed_flops(M, s, tensors):
    """FLOPs the kernel itself executes in one forward: every (packed-row block, key block)
    tile its tile log records as visited, counted whole (QK^T and PV on the MFMA tiles, masked
    elements included), 4 * D * rows * keys each.  One untimed run of the logging variant."""
    q, k, v = tensors
    rb, kb, _ = M.mars_attn_tilelog_geometry(s.batch, s.hq, s.hkv, s.d, s.P, s.L, s.B)
    _, log = M.mars_attn_fwd_tilelog(q, k, v, s.P, s.L, s.B)
    n = int((log > 0).sum().item())
    del log
    return 4.0 * s.d * rb * kb * n


def traffic_from_profile(kernel_tag, src_file):
    """HBM bytes per launch from a committed counter summary, if the kernel source still matches."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_traffic.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m_sha and m_b):
        return None
    sha = hashlib.sha256(open(src_file, "rb").read()).hexdigest()
    return float(m_b.group(1)) if sha == m_sha.group(1) else None


def blas_threads():
    """Threads the oracle's NumPy BLAS actually runs with (the CPU baseline's core count)."""
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline_train(s, budget_s=20.0):
    """fp64 oracle on whole (batch, head) slices of the training layout, FLOP_vt-scaled."""
    from oracle import mars_oracle as O
    from structured_mask_attention_amd import inputs as I
    cores = blas_threads()
    q, k, v = I.train_inputs(s)
    G = s.hq // s.hkv
    qn = q.float().numpy().astype(np.float64)
    kn = k.float().numpy().astype(np.float64)
    vn = v.float().numpy().astype(np.float64)
    vis = O.visible_tile_elems(s.P, s.L, s.B, 128, 128)
    done, t0 = 0, time.perf_counter()
    while done < s.batch * s.hq and time.perf_counter() - t0 < budget_s:
        b, h = divmod(done, s.hq)
        O.attn(qn[b:b + 1, :, h:h + 1], kn[b:b + 1, :, h // G:h // G + 1], vn[b:b + 1, :, h // G:h // G + 1],
               s.P, s.L, s.B)
        done += 1
    dt = time.perf_counter() - t0
    tflops = 4.0 * s.d * vis * done / dt / 1e12
    return {"value": tflops, "unit": "TFLOP/s (visible-tile)", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {s.batch * s.hq} (batch, head) slices of {s.name}, fp64 NumPy, {dt:.1f} s"}


def cpu_baseline_decode(s, budget_s=8.0):
    from oracle import mars_oracle as O
    from structured_mask_attention_amd import inputs as I
    x = I.decode_inputs(s)
    f = lambda t: t.float().numpy().astype(np.float64)
    qw, kw, vw, kc, vc, lg = f(x.q_win), f(x.k_win), f(x.v_win), f(x.k_cache), f(x.v_cache), f(x.logits)
    lens = x.cache_len.numpy()
    seqs, toks, t0 = 0, 0, time.perf_counter()
    while seqs < s.batch and time.perf_counter() - t0 < budget_s:
        b = seqs
        O.decode(qw[b:b + 1], kw[b:b + 1], vw[b:b + 1], kc[b:b + 1], vc[b:b + 1], lens[b:b + 1])
        _, _, n = O.accept(lg[b:b + 1], s.tau)
        toks += int(n.sum())
        seqs += 1
    dt = time.perf_counter() - t0
    return {"value": toks / dt, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{seqs} of {s.batch} sequences of the decode step + accept, fp64 NumPy, {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the MARS hot path here has no multi-GPU mode "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import structured_mask_attention_amd as M
    from structured_mask_attention_amd import inputs as I

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ---- inputs (generated on the host, copied to HBM; `copies` rotated replicas) ----
    st = I.QWEN05B
    sd = I.DECODE7B
    host_t = I.train_inputs(st)
    x = I.decode_inputs(sd)
    host_d = (x.q_win, x.k_win, x.v_win, x.k_cache, x.v_cache, x.cache_len, x.logits)
    ncopy = max(1, args.copies)
    train_sets = [tuple(t.to(dev) for t in host_t) for _ in range(ncopy)]
    dec_sets = [tuple(t.to(dev) for t in host_d) for _ in range(ncopy)]
    q = train_sets[0][0]
    qw = dec_sets[0][0]
    logits = dec_sets[0][6]
    o = torch.empty_like(q)
    od = torch.empty_like(qw)
    dws = torch.empty(M.mars_decode_workspace_bytes(sd.batch, sd.hq, sd.hkv, sd.d, sd.W, sd.cap),
                      dtype=torch.uint8, device=dev)
    aws = torch.empty(M.mars_accept_workspace_bytes(sd.batch, sd.W, sd.vocab, sd.tau), dtype=torch.uint8, device=dev)
    tok = torch.empty((sd.batch, sd.W), dtype=torch.int32, device=dev)
    pmx = torch.empty((sd.batch, sd.W), dtype=torch.float32, device=dev)
    nacc = torch.empty((sd.batch,), dtype=torch.int32, device=dev)
    def attn(i):
        tq, tk, tv = train_sets[i % ncopy]
        M.mars_attn_fwd(tq, tk, tv, st.P, st.L, st.B, out=o)

    def decode(i):
        dq, dk, dv, dkc, dvc, dlen, _ = dec_sets[i % ncopy]
        M.mars_decode_step(dq, dk, dv, dkc, dvc, dlen, out=od, ws=dws)

    def accept(i):
        M.mars_accept(dec_sets[i % ncopy][6], sd.tau, ws=aws, tokens=tok, pmax=pmx, n_accept=nacc)

    def step(i):
        attn(i)
        decode(i)
        accept(i)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # No collector passes inside timed groups: a full pass over torch's objects takes tens
    # of milliseconds and would stall the launching thread.
    gc.collect()
    gc.disable()

    # (1) The timed region: exactly `steps` whole steps, events at its two ends.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    t_step_mean = e0.elapsed_time(e1) * 1e-3 / args.steps

    # (2) Per-kernel durations: each kernel launched `steps` times back to back (same input
    # rotation), events around each group, so launch gaps are amortised as in the trace.
    host_issue = {}

    def group(fn):
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        a.record(stream)
        for i in range(args.steps):
            fn(i)
        z.record(stream)
        host_issue.setdefault(fn.__name__, []).append((time.perf_counter() - h0) / args.steps * 1e6)
        torch.cuda.synchronize()
        return a.elapsed_time(z) * 1e-3 / args.steps

    mgn = torch.empty((sd.batch, sd.W), dtype=torch.float32, device=dev)

    def accept_margin(i):
        M.mars_accept_margin(dec_sets[i % ncopy][6], MARGIN_TAU, ws=aws, tokens=tok, pmax=pmx, margin=mgn,
                             n_accept=nacc)

    reps = [(group(attn), group(decode), group(accept)) for _ in range(3)]
    t_mgn = float(np.mean([group(accept_margin) for _ in range(3)]))
    accept(0)   # leave the probability gate's n_accept in place for the tokens/s figure
    t_attn = np.array([r[0] for r in reps])
    t_dec = np.array([r[1] for r in reps])
    t_acc = np.array([r[2] for r in reps])

    # KV commit (decode loop bookkeeping): timed last, on a scratch cursor array that starts at
    # 0 each group, so it writes cache rows the timed steps above have already read.
    lens_s = torch.zeros_like(dec_sets[0][5])
    valid_s = torch.empty((sd.batch,), dtype=torch.int64, device=dev)
    ovf_s = torch.empty((sd.batch,), dtype=torch.int32, device=dev)

    def commit(i):
        dq_, dk_, dv_, dkc_, dvc_, _, _ = dec_sets[i % ncopy]
        M.mars_kv_commit(dk_, dv_, nacc, dkc_, dvc_, lens_s, valid=valid_s, overflow=ovf_s)

    t_cmt = []
    for _ in range(3):
        lens_s.zero_()
        t_cmt.append(group(commit))
    t_cmt = float(np.mean(t_cmt))

    flop_vt, flop_alg = train_flops(M, st)
    flop_exe = executed_flops(M, st, train_sets[0])
    ta = float(np.mean(t_attn))
    tflops = flop_vt / ta / 1e12
    n_sum = int(nacc.sum().item())
    lens_sum = int(x.cache_len.sum().item())
    dec_bytes = lens_sum * sd.hkv * sd.d * 2 * 2 + (x.q_win.numel() + x.k_win.numel() + x.v_win.numel() + od.numel()) * 2
    acc_bytes = logits.numel() * 2
    td, tc = float(np.mean(t_dec)), float(np.mean(t_acc))

    def time_backward(s2, sets2, reps=10):
        """mars_attn_bwd on a training layout: forward outputs (O, LSE) made once per input
        copy outside the timed region, then `reps` backwards with the same rotation."""
        ws = torch.empty(M.mars_attn_bwd_workspace_bytes(s2.batch, s2.hq, s2.hkv, s2.d, s2.P, s2.L, s2.B),
                         dtype=torch.uint8, device=dev)
        do = I.grad_output(s2).to(dev)
        fw = []
        for tq, tk, tv in sets2:
            lse = torch.empty((s2.batch, s2.hq, s2.N), dtype=torch.float32, device=dev)
            fw.append((M.mars_attn_fwd(tq, tk, tv, s2.P, s2.L, s2.B, lse=lse), lse))
        g = [torch.empty_like(sets2[0][0]), torch.empty_like(sets2[0][1]), torch.empty_like(sets2[0][2])]

        def bwd(r):
            tq, tk, tv = sets2[r % len(sets2)]
            ob, lb = fw[r % len(sets2)]
            M.mars_attn_bwd(tq, tk, tv, ob, lb, do, s2.P, s2.L, s2.B, dq=g[0], dk=g[1], dv=g[2], ws=ws)
        for r in range(3):
            bwd(r)
        a3, z3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a3.record(stream)
        for r in range(reps):
            bwd(r)
        z3.record(stream)
        torch.cuda.synchronize()
        t3 = a3.elapsed_time(z3) * 1e-3 / reps
        fvt, falg = train_flops(M, s2)
        # dQ, dK, dV: five products of the forward's two (S, dP, dV, dK, dQ), same visible tiles
        out = {"workload": s2.name, "us": t3 * 1e6, "tflops_visible_tile": 2.5 * fvt / t3 / 1e12,
               "tflops_alg": 2.5 * falg / t3 / 1e12, "frac_of_peak": 2.5 * fvt / t3 / 1e12 / PEAK_BF16_TFLOPS,
               "workspace_bytes": int(ws.numel())}
        del ws, do, fw, g
        return out

    backward = {}
    if not args.no_backward:
        backward[st.name] = time_backward(st, train_sets)

    # ---- other training layouts (own events, same rotation of input copies) ----
    layouts = {}
    if not args.no_extra_layouts:
        del train_sets, dec_sets
        torch.cuda.empty_cache()
        for s2 in (I.QWEN7B, I.LONG7B):
            h2 = I.train_inputs(s2)
            sets2 = [tuple(t.to(dev) for t in h2) for _ in range(ncopy)]
            q2 = sets2[0][0]
            o2 = torch.empty_like(q2)
            for r in range(3):
                M.mars_attn_fwd(*sets2[r % ncopy], s2.P, s2.L, s2.B, out=o2)
            reps = 10
            a2, z2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a2.record(stream)
            for r in range(reps):
                M.mars_attn_fwd(*sets2[r % ncopy], s2.P, s2.L, s2.B, out=o2)
            z2.record(stream)
            torch.cuda.synchronize()
            t2 = a2.elapsed_time(z2) * 1e-3 / reps
            fvt, falg = train_flops(M, s2)
            fexe = executed_flops(M, s2, sets2[0])
            layouts[s2.name] = {"us": t2 * 1e6, "tflops_visible_tile": fvt / t2 / 1e12,
                                "tflops_alg": falg / t2 / 1e12, "tflops_executed": fexe / t2 / 1e12,
                                "frac_of_peak": fvt / t2 / 1e12 / PEAK_BF16_TFLOPS}
            if not args.no_backward:
                backward[s2.name] = time_backward(s2, sets2, reps=4)
            del sets2, q2, o2
        torch.cuda.empty_cache()

    src = os.path.join(ROOT, "structured_mask_attention_amd", "csrc", "attn_fwd.hip")
    traffic = traffic_from_profile("attn_fwd_bf16_qwen05b", src)
    roofline = {"bound": "mfma", "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / PEAK_BF16_TFLOPS, "traffic": traffic,
                "kernel": "attn_fwd_bf16_kernel<64>", "work_per_launch_flop_vt": flop_vt,
                "achieved_alg": flop_alg / ta / 1e12,
                "work_per_launch_flop_executed": flop_exe, "achieved_executed": flop_exe / ta / 1e12}

    cpu = None
    cpu_dec = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_train(st)
        cpu_dec = cpu_baseline_decode(sd)

    # ---- training loss L_mask + L_AR with its logits gradient (one copy: 6 GB of traffic per
    # call, far beyond the caches) ----
    loss = {}
    if not args.no_loss:
        torch.cuda.empty_cache()
        V = QWEN05B_VOCAB
        lg, tk = I.ce_inputs(st.batch, st.P, st.L, V, 2002, device=dev)
        dlg = torch.empty_like(lg)
        cws = torch.empty(max(16, st.batch * st.N * 4), dtype=torch.uint8, device=dev)
        for _ in range(2):
            M.mars_shifted_ce(lg, tk, st.P, st.L, st.B, grad=True, dlogits=dlg, ws=cws)
        reps = 10
        a4, z4 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a4.record(stream)
        for _ in range(reps):
            M.mars_shifted_ce(lg, tk, st.P, st.L, st.B, grad=True, dlogits=dlg, ws=cws)
        z4.record(stream)
        torch.cuda.synchronize()
        t4 = a4.elapsed_time(z4) * 1e-3 / reps
        ce_bytes = 2 * 2 * st.batch * st.N * V   # bf16 logits read once, bf16 gradient written once
        loss = {"workload": f"{st.name}_V{V}", "us": t4 * 1e6, "GBps": ce_bytes / t4 / 1e9,
                "frac_hbm": ce_bytes / t4 / 1e9 / PEAK_HBM_GBS, "bytes": ce_bytes}
        del lg, tk, dlg, cws

    rec = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step_mean * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes of the Qwen2.5 workloads; no weights or datasets)",
        "config": {"workload": st.name, "decode_workload": sd.name, "global_batch": st.batch, "seq_len": st.N,
                   "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "decode": {
            "tokens_per_s": n_sum / (td + tc),
            "tokens_accepted": n_sum,
            "decode_us": td * 1e6, "accept_us": tc * 1e6,
            "decode_us_groups": [float(t) * 1e6 for t in t_dec],
            "decode_GBps": dec_bytes / td / 1e9, "decode_frac_hbm": dec_bytes / td / 1e9 / PEAK_HBM_GBS,
            "accept_GBps": acc_bytes / tc / 1e9, "accept_frac_hbm": acc_bytes / tc / 1e9 / PEAK_HBM_GBS,
            "accept_margin_us": t_mgn * 1e6, "accept_margin_GBps": acc_bytes / t_mgn / 1e9,
            "accept_margin_tau": MARGIN_TAU,
            "kv_commit_us": t_cmt * 1e6,
            "tokens_per_s_with_commit": n_sum / (td + tc + t_cmt),
            "cpu_baseline": cpu_dec,
        },
        "train_attn_us": ta * 1e6,
        "train_attn_us_groups": [float(t) * 1e6 for t in t_attn],
        "train_layouts": layouts,
        "train_backward": backward,
        "train_loss": loss,
        "wall_s_timed_region": t_wall,
        "host_issue_us_per_call": {k: [round(x, 1) for x in v] for k, v in host_issue.items()},
        "input_copies_rotated": ncopy,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
