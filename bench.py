#!/usr/bin/env python3
"""Benchmark of the MARS hot path on one MI355X.

One step = one pass of the whole path on synthetic, seeded inputs resident in HBM:
  1. mars_attn_fwd on the long 7B-shaped training layout (batch 1, 28/4 heads, head_dim 128,
     P=1024, L=7168, B=32: N = 15360), the largest training layout that fits one GPU;
  2. mars_decode_step on the Qwen2.5-7B-shaped decode workload (32 sequences, 28/4 heads,
     head_dim 128, cache lengths U[512, 4096], 4 window rows);
  3. mars_accept on its logits [32, 4, 152064] at tau = 0.95.
The timed region is exactly K whole steps, with HIP events (on the launch stream) at its two
ends and between the three launches of every step, so each kernel's average duration over the
timed region comes from the same run.  `value` is the forward's visible-tile TFLOP/s over that
average; `roofline` is the forward against the bf16 MFMA peak on its algorithmic FLOPs
(4 * head_dim * visible (query, key) pairs of the mask, per query head and batch), with the
visible-tile and executed-tile figures beside it.
Every kernel is also launched >= 50 more times alone, one event pair per launch, for the
median and the 10th/90th percentiles; the 0.5B- and 7B-shaped training layouts get their own
roofline blocks from such samples, and so do the backward (mars_attn_bwd), the margin gate,
the KV commit and the training loss (mars_shifted_ce).  Three independent copies of every
input rotate across launches, so the 256 MB Infinity Cache holds none of a launch's inputs.
The CPU baseline is the fp64 oracle on a bounded sample of each workload, timed on this host.

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
SAMPLE_LAUNCHES = 50          # launches per kernel for the median / percentiles


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
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


def traffic_from_profile(tag, src_file):
    """HBM bytes per launch from a committed counter summary (profiles/<tag>_traffic.md), if
    the kernel source still matches the one the counters were taken on."""
    path = os.path.join(ROOT, "profiles", f"{tag}_traffic.md")
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


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def stats_us(samples_s):
    a = np.asarray(samples_s) * 1e6
    return {"median_us": float(np.median(a)), "p10_us": float(np.percentile(a, 10)),
            "p90_us": float(np.percentile(a, 90)), "mean_us": float(a.mean()), "n": int(a.size)}


def cpu_baseline_train(s, budget_s):
    """fp64 oracle on whole (batch, query head) slices of a training layout, until the budget
    is spent (at least one slice); throughput on the slices' algorithmic FLOPs."""
    from oracle import mars_oracle as O
    from structured_mask_attention_amd import inputs as I
    q, k, v = I.train_inputs(s)
    G = s.hq // s.hkv
    f = lambda t: t.float().numpy().astype(np.float64)
    qn, kn, vn = f(q), f(k), f(v)
    nnz = O.mask_nnz(s.P, s.L, s.B)
    done, t0 = 0, time.perf_counter()
    total = s.batch * s.hq
    while done < total and (done == 0 or time.perf_counter() - t0 < budget_s):
        b, h = divmod(done, s.hq)
        O.attn(qn[b:b + 1, :, h:h + 1], kn[b:b + 1, :, h // G:h // G + 1], vn[b:b + 1, :, h // G:h // G + 1],
               s.P, s.L, s.B)
        done += 1
    dt = time.perf_counter() - t0
    flop = 4.0 * s.d * nnz * done
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s (algorithmic: 4·D·visible pairs)",
            "gflops_alg": flop / dt / 1e9, "cores": blas_threads(), "cpu": cpu_model(), "kind": "oracle",
            "seconds": dt, "sample": f"{done} of {total} (batch, head) slices of {s.name}, fp64 NumPy"}


def cpu_baseline_decode(s, budget_s):
    """fp64 oracle decode step + acceptance, sequence by sequence, until the budget is spent."""
    from oracle import mars_oracle as O
    from structured_mask_attention_amd import inputs as I
    x = I.decode_inputs(s)
    f = lambda t: t.float().numpy().astype(np.float64)
    qw, kw, vw, kc, vc, lg = f(x.q_win), f(x.k_win), f(x.v_win), f(x.k_cache), f(x.v_cache), f(x.logits)
    lens = x.cache_len.numpy()
    seqs, toks, t0 = 0, 0, time.perf_counter()
    while seqs < s.batch and (seqs == 0 or time.perf_counter() - t0 < budget_s):
        b = seqs
        O.decode(qw[b:b + 1], kw[b:b + 1], vw[b:b + 1], kc[b:b + 1], vc[b:b + 1], lens[b:b + 1])
        _, _, n = O.accept(lg[b:b + 1], s.tau)
        toks += int(n.sum())
        seqs += 1
    dt = time.perf_counter() - t0
    return {"value": toks / dt, "unit": "tokens/s", "cores": blas_threads(), "cpu": cpu_model(), "kind": "oracle",
            "seconds": dt, "sample": f"{seqs} of {s.batch} sequences of the decode step + accept, fp64 NumPy"}


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
    ncopy = max(1, args.copies)
    Ev = lambda: torch.cuda.Event(enable_timing=True)

    # ---- inputs (generated on the host, copied to HBM; `ncopy` rotated replicas) ----
    st = I.LONG7B
    sd = I.DECODE7B
    host_t = I.train_inputs(st)
    x = I.decode_inputs(sd)
    host_d = (x.q_win, x.k_win, x.v_win, x.k_cache, x.v_cache, x.cache_len, x.logits)
    train_sets = [tuple(t.to(dev) for t in host_t) for _ in range(ncopy)]
    dec_sets = [tuple(t.to(dev) for t in host_d) for _ in range(ncopy)]
    o = torch.empty_like(train_sets[0][0])
    od = torch.empty_like(dec_sets[0][0])
    dws = torch.empty(M.mars_decode_workspace_bytes(sd.batch, sd.hq, sd.hkv, sd.d, sd.W, sd.cap),
                      dtype=torch.uint8, device=dev)
    aws = torch.empty(M.mars_accept_workspace_bytes(sd.batch, sd.W, sd.vocab, sd.tau), dtype=torch.uint8, device=dev)
    tok = torch.empty((sd.batch, sd.W), dtype=torch.int32, device=dev)
    pmx = torch.empty((sd.batch, sd.W), dtype=torch.float32, device=dev)
    mgn = torch.empty((sd.batch, sd.W), dtype=torch.float32, device=dev)
    nacc = torch.empty((sd.batch,), dtype=torch.int32, device=dev)

    def attn(i):
        tq, tk, tv = train_sets[i % ncopy]
        M.mars_attn_fwd(tq, tk, tv, st.P, st.L, st.B, out=o)

    def decode(i):
        dq, dk, dv, dkc, dvc, dlen, _ = dec_sets[i % ncopy]
        M.mars_decode_step(dq, dk, dv, dkc, dvc, dlen, out=od, ws=dws)

    def accept(i):
        M.mars_accept(dec_sets[i % ncopy][6], sd.tau, ws=aws, tokens=tok, pmax=pmx, n_accept=nacc)

    def accept_margin(i):
        M.mars_accept_margin(dec_sets[i % ncopy][6], MARGIN_TAU, ws=aws, tokens=tok, pmax=pmx, margin=mgn,
                             n_accept=nacc)

    for i in range(args.warmup):
        attn(i)
        decode(i)
        accept(i)
    torch.cuda.synchronize()
    # No collector passes inside timed regions: a full pass over torch's objects takes tens
    # of milliseconds and would stall the launching thread.
    gc.collect()
    gc.disable()

    # (1) The timed region: exactly `steps` whole steps; events at its ends and between the
    # launches of each step (all on the launch stream).
    ev = [[Ev() for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        attn(i)
        ev[i][1].record(stream)
        decode(i)
        ev[i][2].record(stream)
        accept(i)
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    t_step = ev[0][0].elapsed_time(ev[-1][3]) * 1e-3 / args.steps
    tr_attn = [e[0].elapsed_time(e[1]) * 1e-3 for e in ev]
    tr_dec = [e[1].elapsed_time(e[2]) * 1e-3 for e in ev]
    tr_acc = [e[2].elapsed_time(e[3]) * 1e-3 for e in ev]
    n_sum = int(nacc.sum().item())

    # (2) Per-kernel samples: each kernel launched >= SAMPLE_LAUNCHES times alone (same input
    # rotation), one event pair per launch.
    nsamp = max(SAMPLE_LAUNCHES, args.steps)
    host_issue = {}

    def sample(fn, n=nsamp, setup=None, name=None):
        pairs = [(Ev(), Ev()) for _ in range(n)]
        torch.cuda.synchronize()
        h0 = time.perf_counter()
        for i in range(n):
            if setup is not None:
                setup(i)
            pairs[i][0].record(stream)
            fn(i)
            pairs[i][1].record(stream)
        host_issue[name or fn.__name__] = round((time.perf_counter() - h0) / n * 1e6, 1)
        torch.cuda.synchronize()
        return [a.elapsed_time(z) * 1e-3 for a, z in pairs]

    s_attn = sample(attn, name=f"attn_fwd {st.name}")
    s_dec = sample(decode)
    s_acc = sample(accept)
    s_mgn = sample(accept_margin)
    accept(0)   # leave the probability gate's n_accept in place for the commit timing

    # KV commit (decode loop bookkeeping): on a scratch cursor array that starts at 0 for each
    # launch, so it writes cache rows the steps above have already read.
    lens_s = torch.zeros_like(dec_sets[0][5])
    valid_s = torch.empty((sd.batch,), dtype=torch.int64, device=dev)
    ovf_s = torch.empty((sd.batch,), dtype=torch.int32, device=dev)

    def kv_commit(i):
        _, dk_, dv_, dkc_, dvc_, _, _ = dec_sets[i % ncopy]
        M.mars_kv_commit(dk_, dv_, nacc, dkc_, dvc_, lens_s, valid=valid_s, overflow=ovf_s)

    s_cmt = sample(kv_commit, setup=lambda i: lens_s.zero_())

    flop_vt, flop_alg = train_flops(M, st)
    flop_exe = executed_flops(M, st, train_sets[0])
    ta = float(np.mean(tr_attn))
    lens_sum = int(x.cache_len.sum().item())
    dec_bytes = lens_sum * sd.hkv * sd.d * 2 * 2 + (x.q_win.numel() + x.k_win.numel() + x.v_win.numel() + od.numel()) * 2
    acc_bytes = dec_sets[0][6].numel() * 2
    td, tc = float(np.mean(tr_dec)), float(np.mean(tr_acc))
    src_fwd = os.path.join(ROOT, "structured_mask_attention_amd", "csrc", "attn_fwd.hip")

    def fwd_roofline(s, t_avg, samples, fvt, falg, fexe, kernel):
        return {"bound": "mfma", "achieved": falg / t_avg / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": falg / t_avg / 1e12 / PEAK_BF16_TFLOPS,
                "traffic": traffic_from_profile(f"attn_fwd_{s.name}", src_fwd),
                "kernel": kernel, "workload": s.name,
                "work_per_launch_flop_alg": falg, "work_per_launch_flop_vt": fvt,
                "work_per_launch_flop_executed": fexe,
                "achieved_vt": fvt / t_avg / 1e12, "frac_vt": fvt / t_avg / 1e12 / PEAK_BF16_TFLOPS,
                "achieved_executed": fexe / t_avg / 1e12, "avg_us": t_avg * 1e6,
                "launches": stats_us(samples)}

    roofline = fwd_roofline(st, ta, s_attn, flop_vt, flop_alg, flop_exe, "attn_fwd_bf16_kernel<128, false>")
    roofline["avg_over"] = f"the {args.steps} forwards of the timed region (event pair around each launch)"

    def time_backward(s2, sets2, n=nsamp):
        """mars_attn_bwd on a training layout: forward outputs (O, LSE) made once per input
        copy outside the sample, then `n` backwards with the same rotation."""
        ws = torch.empty(M.mars_attn_bwd_workspace_bytes(s2.batch, s2.hq, s2.hkv, s2.d, s2.P, s2.L, s2.B),
                         dtype=torch.uint8, device=dev)
        do = I.grad_output(s2).to(dev)
        fw = []
        for tq, tk, tv in sets2:
            lse = torch.empty((s2.batch, s2.hq, s2.N), dtype=torch.float32, device=dev)
            fw.append((M.mars_attn_fwd(tq, tk, tv, s2.P, s2.L, s2.B, lse=lse), lse))
        g = [torch.empty_like(sets2[0][0]), torch.empty_like(sets2[0][1]), torch.empty_like(sets2[0][2])]

        def attn_bwd(r):
            tq, tk, tv = sets2[r % len(sets2)]
            ob, lb = fw[r % len(sets2)]
            M.mars_attn_bwd(tq, tk, tv, ob, lb, do, s2.P, s2.L, s2.B, dq=g[0], dk=g[1], dv=g[2], ws=ws)
        for r in range(3):
            attn_bwd(r)
        smp = sample(attn_bwd, n, name=f"attn_bwd {s2.name}")
        t3 = float(np.median(smp))
        fvt, falg = train_flops(M, s2)
        # dQ, dK, dV: five products of the forward's two (S, dP, dV, dK, dQ), same visible pairs
        out = {"workload": s2.name, "bound": "mfma", "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
               "achieved": 2.5 * falg / t3 / 1e12, "frac": 2.5 * falg / t3 / 1e12 / PEAK_BF16_TFLOPS,
               "achieved_vt": 2.5 * fvt / t3 / 1e12, "work_per_launch_flop_alg": 2.5 * falg,
               "launches": stats_us(smp), "workspace_bytes": int(ws.numel())}
        del ws, do, fw, g
        return out

    backward = {}
    if not args.no_backward:
        backward[st.name] = time_backward(st, train_sets)

    # ---- the other training layouts (per-launch samples, same rotation of input copies) ----
    layouts = {st.name: roofline}
    if not args.no_extra_layouts:
        del train_sets
        torch.cuda.empty_cache()
        for s2 in (I.QWEN7B, I.QWEN05B):
            h2 = I.train_inputs(s2)
            sets2 = [tuple(t.to(dev) for t in h2) for _ in range(ncopy)]
            o2 = torch.empty_like(sets2[0][0])

            def attn_fwd(r, sets2=sets2, s2=s2, o2=o2):
                M.mars_attn_fwd(*sets2[r % ncopy], s2.P, s2.L, s2.B, out=o2)
            for r in range(3):
                attn_fwd(r)
            smp = sample(attn_fwd, name=f"attn_fwd {s2.name}")
            fvt, falg = train_flops(M, s2)
            fexe = executed_flops(M, s2, sets2[0])
            kern = f"attn_fwd_bf16_kernel<{s2.d}, false>"
            layouts[s2.name] = fwd_roofline(s2, float(np.median(smp)), smp, fvt, falg, fexe, kern)
            layouts[s2.name]["avg_over"] = f"median of {len(smp)} single launches"
            if not args.no_backward:
                backward[s2.name] = time_backward(s2, sets2)
            del sets2, o2
        torch.cuda.empty_cache()

    # ---- training loss L_mask + L_AR with its logits gradient (one copy: 6 GB of traffic per
    # call, far beyond the caches) ----
    loss = {}
    if not args.no_loss:
        del dec_sets
        torch.cuda.empty_cache()
        s5 = I.QWEN05B
        V = QWEN05B_VOCAB
        lg, tk = I.ce_inputs(s5.batch, s5.P, s5.L, V, 2002, device=dev)
        dlg = torch.empty_like(lg)
        cws = torch.empty(max(16, s5.batch * s5.N * 4), dtype=torch.uint8, device=dev)

        def shifted_ce(_):
            M.mars_shifted_ce(lg, tk, s5.P, s5.L, s5.B, grad=True, dlogits=dlg, ws=cws)
        for _ in range(2):
            shifted_ce(0)
        smp = sample(shifted_ce, 20)
        t4 = float(np.median(smp))
        ce_bytes = 2 * 2 * s5.batch * s5.N * V   # bf16 logits read once, bf16 gradient written once
        loss = {"workload": f"{s5.name}_V{V}", "bound": "hbm", "achieved": ce_bytes / t4 / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": ce_bytes / t4 / 1e9 / PEAK_HBM_GBS, "bytes": ce_bytes,
                "launches": stats_us(smp)}
        del lg, tk, dlg, cws

    cpu = None
    cpu_all = {}
    if not args.no_cpu_baseline:
        cpu = cpu_baseline_train(st, budget_s=12.0)
        cpu_all[st.name] = cpu
        cpu_all[I.QWEN7B.name] = cpu_baseline_train(I.QWEN7B, budget_s=5.0)
        cpu_all[I.QWEN05B.name] = cpu_baseline_train(I.QWEN05B, budget_s=6.0)
        cpu_all[I.TINY.name] = cpu_baseline_train(I.TINY, budget_s=1.0)
        cpu_all[sd.name] = cpu_baseline_decode(sd, budget_s=6.0)

    def hbm(name, t_avg, samples, nbytes, extra=None):
        r = {"bound": "hbm", "achieved": nbytes / t_avg / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": nbytes / t_avg / 1e9 / PEAK_HBM_GBS, "bytes": nbytes, "avg_us": t_avg * 1e6,
             "launches": stats_us(samples)}
        if extra:
            r.update(extra)
        return r

    rec = {
        "metric": METRIC,
        "value": flop_vt / ta / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes of the Qwen2.5 workloads; no weights or datasets)",
        "config": {"workload": st.name, "decode_workload": sd.name, "global_batch": st.batch, "seq_len": st.N,
                   "parallelism": "none (1 GPU)",
                   "step": "mars_attn_fwd (long layout) + mars_decode_step + mars_accept (7B decode workload)"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "decode": {
            "tokens_per_s": n_sum / (td + tc),
            "tokens_accepted": n_sum,
            "decode_step": hbm("decode", td, s_dec, dec_bytes,
                               {"avg_over": f"the {args.steps} decode steps of the timed region"}),
            "accept": hbm("accept", tc, s_acc, acc_bytes,
                          {"avg_over": f"the {args.steps} accept calls of the timed region"}),
            "accept_margin": hbm("accept_margin", float(np.median(s_mgn)), s_mgn, acc_bytes,
                                 {"tau": MARGIN_TAU, "avg_over": "median of single launches"}),
            "kv_commit": {"launches": stats_us(s_cmt)},
            "tokens_per_s_with_commit": n_sum / (td + tc + float(np.median(s_cmt))),
            "tokens_per_step_fixed_n1": sd.batch,
            "steps_per_s": 1.0 / (td + tc),
        },
        "train_layouts": layouts,
        "train_backward": backward,
        "train_loss": loss,
        "cpu_baselines": cpu_all,
        "wall_s_timed_region": t_wall,
        "host_issue_us_per_call": host_issue,
        "input_copies_rotated": ncopy,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
