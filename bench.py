"""Throughput of ReHyAt hybrid attention on one MI355X (librehyat, bf16 MFMA).

Workload (the metric's configuration): the 21x30x52 latent of a 5 s 480x832 video,
batch 2 (cond/uncond), 12 heads, D = F = 128, chunks of Tc = 3 frames with To = 1 overlap
frame, causal form; bf16 q, k, v, W with fp32 accumulation and fp32 output; synthetic
seeded inputs with a per-head scale (synthetic/__init__.py).

A step is one call of rehyat_hybrid_fwd (causal): phi(k) and the per-frame state sums,
the exclusive scan to the per-chunk states, then the attention kernel (phi(q), linear
read-out, windowed softmax and joint normalisation fused). Inputs are resident in HBM.

Printed JSON line: tokens/s (value), ms per step, TFLOP/s and fraction of the bf16 MFMA
peak over the whole step, the roofline of the dominant kernel (the attention kernel,
timed with HIP events recorded by the library on its launch stream), the float64 CPU
oracle timed on a bounded sample (cpu_baseline), and context timings: the same step with
the learned polynomial feature map and with 1 + elu, as 7 recurrent steps, the
bidirectional form, and full softmax attention of the same shape (one chunk covering the
whole sequence) with librehyat and with torch's SDPA.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline] [--no-context]
    python bench.py --phi mlp|elu   the same line with another feature map of key design 3
    python bench.py --workload c2|c5   the same line for the 21x20x30 bidirectional (320x480)
                                or the 49x30x52 wide-chunk (Tc 7, To 3, F 256) workload
    python bench.py --sweep     (Tc, To) grid of the ablation, one JSON line per entry
    python bench.py --bwd       the backward of the causal form on the same workload
    python bench.py --stream    the 81x30x52 streaming workload: 27 single-launch recurrent
                                steps per pass (chunks resident in HBM)
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "hybrid-attn tokens/s & TFLOP/s per MI355X at 21×30×52, % of MFMA peak"
COPY_BYTES = 256 << 20
KERNEL_SOURCE = os.path.join(ROOT, "hybrid_softmax_linear_amd", "csrc", "attn_bf16.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hybrid_attn_bf16_c3_traffic.json")


def measured_traffic():
    """HBM bytes per launch of the attention kernel from the committed counter summary,
    or None when that summary was taken on a different kernel source."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        with open(KERNEL_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec.get("traffic_bytes_per_launch")


MFMA_PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16: 256 CU x 4096 flop/clk x 2.4 GHz
HBM_PEAK_GBS = 8000.0


def attn_kernel_name(cfg, F):
    """The bf16 attention kernel a whole-sequence launch runs: the persistent form (one
    workgroup per compute unit) from 4 query tiles of 256 rows per compute unit."""
    import torch
    Np = cfg.Tc * cfg.HW
    nch = -(-cfg.T // cfg.Tc)
    last = cfg.T * cfg.HW - (nch - 1) * Np
    tiles = cfg.B * cfg.H * ((nch - 1) * (-(-Np // 256)) + -(-last // 256))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return f"hybrid_attn_bf16_kernel<{F}, {'true' if tiles >= 4 * cus else 'false'}>"


def flop_model(B, H, T, HW, D, F, Tc, To, causal=True, phi_row_flop=None):
    """Algorithmic FLOPs (only what the method needs: no padding, no masked pairs).

    window pairs: 4*D each (q.k and p*v); phi(q), phi(k): phi_row_flop per row each (the
    fixed map's u = x W: 2*D*F; the learned map: 2*D*h + 2*h*F; 1 + elu: 0); linear
    read-out phi(q) S: 2*F*D per query row with a non-empty linear set; state phi(k)^T v:
    2*F*D per key that enters some linear set.
    Returns (total, attention-kernel part, state-kernel part, window pairs per head).
    """
    pf = 2 * D * F if phi_row_flop is None else phi_row_flop
    N, Np = T * HW, Tc * HW
    pairs = rows_lin = 0
    t = 0
    while t * Np < N:
        r0, r1 = t * Np, min((t + 1) * Np, N)
        lo, hi = max(t * Np - To * HW, 0), r1
        pairs += (r1 - r0) * (hi - lo)
        if lo > 0 or (not causal and hi < N):
            rows_lin += r1 - r0
        t += 1
    last_lo = max((t - 1) * Np - To * HW, 0)
    keys_state = N if not causal else last_lo
    attn = 4 * D * pairs + pf * rows_lin + 2 * F * D * rows_lin
    state = pf * keys_state + 2 * F * D * keys_state
    BH = B * H
    return BH * (attn + state), BH * attn, BH * state, pairs


def flop_model_bwd(B, H, T, HW, D, F, Tc, To):
    """Algorithmic FLOPs of the causal backward (fixed map).

    window pairs: 10*D each (the scores again, dP = dy.v, and the dq, dk, dv products);
    query rows with a linear set: 10*D*F (phi(q), S g, W gq, dWq, and the reverse state
    phi(q) g^T); keys in some linear set: 12*D*F (phi(k), the forward state phi(k)^T v,
    G v, G^T phi(k), W gk, dWk). Returns (total, dk/dv-kernel part, dq-kernel part).
    """
    N, Np = T * HW, Tc * HW
    pairs = rows_lin = 0
    t = 0
    while t * Np < N:
        r0, r1 = t * Np, min((t + 1) * Np, N)
        lo = max(t * Np - To * HW, 0)
        pairs += (r1 - r0) * (r1 - lo)
        rows_lin += (r1 - r0) if lo > 0 else 0
        t += 1
    keys_lin = max((t - 1) * Np - To * HW, 0)
    BH = B * H
    total = BH * (10 * D * pairs + 10 * D * F * rows_lin + 12 * D * F * keys_lin)
    dkdv = BH * (8 * D * pairs + 8 * D * F * keys_lin)     # as the dk/dv kernel runs them
    dq = BH * (6 * D * pairs + 6 * D * F * rows_lin)       # as the dq kernel runs them
    return total, dkdv, dq


def bench_bwd(args):
    """One line for the backward: rehyat_hybrid_bwd at 21x30x52 (y, lse resident)."""
    import torch
    import synthetic as syn
    import hybrid_softmax_linear_amd as hs
    from hybrid_softmax_linear_amd import torch_api as ta
    cfg = syn.config(3)
    inp = syn.make_inputs(cfg)
    dev = torch.device("cuda:0")
    q, k, v, W = (inp[n].to(dev) for n in ("q", "k", "v", "W"))
    dy = syn.make_upstream(tuple(q.shape), seed=cfg.seed, dtype="f32").to(dev)
    desc = hs.Desc(B=cfg.B, H=cfg.H, T=cfg.T, HW=cfg.HW, D=cfg.D, F=cfg.F, Tc=cfg.Tc, To=cfg.To,
                   dtype=hs.BF16, y_dtype=hs.F32, mode=hs.CAUSAL)
    stream = torch.cuda.current_stream().cuda_stream
    y = torch.empty(q.shape, dtype=torch.float32, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    wsf = ta.workspace(hs.rehyat_hybrid_fwd_workspace(desc), dev)
    hs.rehyat_hybrid_fwd_stats(desc, q, k, v, W, W, y, lse, wsf, stream=stream)
    f32 = dict(dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty(q.shape, **f32) for _ in range(3))
    dWq, dWk = torch.empty(W.shape, **f32), torch.empty(W.shape, **f32)
    ws = ta.workspace(hs.rehyat_hybrid_bwd_workspace(desc), dev)

    def step():
        hs.rehyat_hybrid_bwd(desc, q, k, v, W, W, y, lse, dy, dq, dk, dv, dWq, dWk, ws,
                             stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    times = {}
    for kern, name in ((2, "dkdv"), (3, "dq")):
        hs.rehyat_timing_enable(True, kern)
        ms = time_calls(step, args.steps, 0)
        kms, n = hs.rehyat_timing_read()
        hs.rehyat_timing_enable(False)
        times[name] = (kms / max(n, 1), n, ms)
    ms = min(t[2] for t in times.values())
    total, f_dkdv, f_dq = flop_model_bwd(cfg.B, cfg.H, cfg.T, cfg.HW, cfg.D, cfg.F, cfg.Tc, cfg.To)
    dk_ms, dk_n, _ = times["dkdv"]
    dq_ms, dq_n, _ = times["dq"]
    fwd_ms = time_calls(lambda: hs.rehyat_hybrid_fwd_stats(desc, q, k, v, W, W, y, lse, wsf,
                                                            stream=stream), max(3, args.steps // 2), 2)
    tokens = cfg.B * cfg.N
    result = {
        "metric": "hybrid-attn backward tokens/s & TFLOP/s per MI355X at 21×30×52",
        "value": tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "21x30x52 latent (480x832, 5 s): B2 H12 D128 F128, Tc3 To1, causal, "
                               "one rehyat_hybrid_bwd call per step (y, lse and dy resident)",
                   "global_batch": cfg.B, "seq_len": cfg.N, "parallelism": "none (1 GPU)"},
        "tflops": total / (ms * 1e-3) / 1e12,
        "mfma_peak_frac": total / (ms * 1e-3) / 1e12 / MFMA_PEAK_BF16_TFLOPS,
        "flop_per_step": total,
        "roofline": {"bound": "mfma", "kernel": "bwd_dkdv_kernel<128>",
                     "achieved": f_dkdv / (dk_ms * 1e-3) / 1e12, "peak": MFMA_PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s",
                     "frac": f_dkdv / (dk_ms * 1e-3) / 1e12 / MFMA_PEAK_BF16_TFLOPS,
                     "traffic": None, "flop_per_launch": f_dkdv, "avg_launch_ms": dk_ms,
                     "launches_timed": dk_n},
        "cpu_baseline": None,
        "context": {"dq_kernel_ms": dq_ms, "dq_kernel_tflops": f_dq / (dq_ms * 1e-3) / 1e12,
                    "fwd_stats_ms": fwd_ms, "fwd_plus_bwd_ms": fwd_ms + ms},
    }
    print(json.dumps(result))
    return 0


def bench_stream(args):
    """One line for streaming: 27 recurrent steps over the 81x30x52 latent (B1 H12, Tc3 To1),
    each step's q, k, v chunk resident in HBM; a pass is the 27 steps, each one launch of
    rehyat_recurrent_step_fused. Context: the same pass with rehyat_recurrent_step (six
    launches per step), and the pass with each chunk copied from pinned host memory before
    its step (PCIe-inclusive; the copies alone are timed too)."""
    import torch
    import synthetic as syn
    import hybrid_softmax_linear_amd as hs
    from hybrid_softmax_linear_amd import torch_api as ta
    cfg = syn.config(4)
    inp = syn.make_inputs(cfg)
    dev = torch.device("cuda:0")
    Np = cfg.Tc * cfg.HW
    W = inp["W"].to(dev)
    chunks = [tuple(inp[n][:, :, t * Np:(t + 1) * Np].contiguous().to(dev) for n in ("q", "k", "v"))
              for t in range(cfg.n_chunks)]
    del inp
    yc = torch.empty(chunks[0][0].shape, dtype=torch.float32, device=dev)
    steps = cfg.n_chunks

    def timed(fused, kernel):
        rec = ta.Recurrent(cfg.B, cfg.H, cfg.D, cfg.F, T=cfg.T, HW=cfg.HW, Tc=cfg.Tc, To=cfg.To,
                           device=dev, fused=fused)

        def one_pass():
            rec.t = 0
            for (qc, kc, vc) in chunks:
                rec.step(qc, kc, vc, W, out=yc)

        for _ in range(args.warmup):
            one_pass()
        torch.cuda.synchronize()
        hs.rehyat_timing_enable(True, kernel)
        ms = time_calls(one_pass, args.steps, 0)
        kms, n = hs.rehyat_timing_read()
        hs.rehyat_timing_enable(False)
        return ms, kms / max(n, 1), n

    ms, step_ms, n = timed(True, 4)
    ms_multi, attn_ms_multi, _ = timed(False, 1)

    # PCIe-inclusive pass: each chunk copied from pinned host memory into fixed device
    # buffers before its step, on the same stream (context only; inputs are not resident)
    host = [tuple(x.cpu().pin_memory() for x in c) for c in chunks]
    bufs = tuple(torch.empty_like(x) for x in chunks[0])
    rec = ta.Recurrent(cfg.B, cfg.H, cfg.D, cfg.F, T=cfg.T, HW=cfg.HW, Tc=cfg.Tc, To=cfg.To,
                       device=dev, fused=True)

    def h2d_pass(with_step=True):
        rec.t = 0
        for hc in host:
            for b, h in zip(bufs, hc):
                b.copy_(h, non_blocking=True)
            if with_step:
                rec.step(*bufs, W, out=yc)

    for _ in range(2):
        h2d_pass()
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    ms_h2d = time_calls(h2d_pass, max(3, args.steps // 4), 0)
    ms_copy = time_calls(lambda: h2d_pass(False), max(3, args.steps // 4), 0)
    free1 = torch.cuda.mem_get_info()[0]
    chunk_bytes = sum(x.numel() * x.element_size() for x in chunks[0])
    del host, bufs, rec
    total, attn_total = flop_model(cfg.B, cfg.H, cfg.T, cfg.HW, cfg.D, cfg.F, cfg.Tc, cfg.To)[:2]
    per_launch = total / steps
    result = {
        "metric": "hybrid-attn streaming tokens/s per MI355X at 81×30×52",
        "value": cfg.B * cfg.N / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "81x30x52 latent: B1 H12 D128 F128, Tc3 To1, causal, 27 "
                               "rehyat_recurrent_step_fused calls per step (one pass over the "
                               "video)",
                   "global_batch": cfg.B, "seq_len": cfg.N, "parallelism": "none (1 GPU)"},
        "tflops": total / (ms * 1e-3) / 1e12,
        "mfma_peak_frac": total / (ms * 1e-3) / 1e12 / MFMA_PEAK_BF16_TFLOPS,
        "flop_per_step": total,
        "roofline": {"bound": "mfma", "kernel": "recurrent_step_bf16_kernel<128>",
                     "achieved": per_launch / (step_ms * 1e-3) / 1e12,
                     "peak": MFMA_PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": per_launch / (step_ms * 1e-3) / 1e12 / MFMA_PEAK_BF16_TFLOPS,
                     "traffic": None, "flop_per_launch": per_launch,
                     "avg_launch_ms": step_ms, "launches_timed": n},
        "cpu_baseline": None,
        "context": {"ms_per_recurrent_step": ms / steps,
                    "multi_launch_ms_per_pass": ms_multi,
                    "multi_launch_ms_per_step": ms_multi / steps,
                    "multi_launch_attention_kernel_ms": attn_ms_multi,
                    "multi_launch_attention_tflops": attn_total / steps / (attn_ms_multi * 1e-3) / 1e12,
                    "single_over_multi_launch_speedup": ms_multi / ms,
                    "pcie_inclusive_ms_per_step": ms_h2d / steps,
                    "pcie_inclusive_tokens_per_s": cfg.B * cfg.N / (ms_h2d * 1e-3),
                    "h2d_copy_ms_per_step": ms_copy / steps,
                    "h2d_copy_GB_per_s": chunk_bytes / (ms_copy / steps * 1e-3) / 1e9,
                    "device_free_bytes_change_over_pcie_passes": free1 - free0},
    }
    print(json.dumps(result))
    return 0


# ---- CPU baseline: the float64 oracle on a bounded sample --------------------------------

def _oracle_head(args):
    from threadpoolctl import threadpool_limits
    import oracle as orc
    q, k, v, W, HW, Tc, To = args
    with threadpool_limits(1):
        t0 = time.perf_counter()
        orc.hybrid_attention(q, k, v, W, W, HW=HW, Tc=Tc, To=To, causal=True)
        return time.perf_counter() - t0


def cpu_baseline(inp, cfg):
    """Time the oracle on whole heads of the workload, one head per worker process.

    Runs before the GPU is touched (worker processes are forked). Returns the
    cpu_baseline JSON object, in tokens/s of the full workload."""
    import multiprocessing as mp
    import synthetic as syn
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(cores, 16, cfg.B * cfg.H))
    W = syn.to_f64(inp["W"])
    jobs = []
    for i in range(workers):
        b, h = divmod(i, cfg.H)
        jobs.append((syn.to_f64(inp["q"][b, h]), syn.to_f64(inp["k"][b, h]),
                     syn.to_f64(inp["v"][b, h]), W, cfg.HW, cfg.Tc, cfg.To))
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(workers) as pool:
        per_head = pool.map(_oracle_head, jobs)
    wall = time.perf_counter() - t0
    heads_total = cfg.B * cfg.H
    # whole workload = B*N tokens through all B*H heads, at the sampled rate
    tokens_per_s = cfg.B * cfg.N / (wall * heads_total / workers)
    return {"value": tokens_per_s, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{workers} of {heads_total} heads of the same workload (all {cfg.N} query "
                      f"rows each), one head per process, 1 BLAS thread each; wall {wall:.1f} s, "
                      f"mean {sum(per_head) / len(per_head):.1f} s per head; scaled to all heads",
            "host_cores_visible": cores, "cpu_model": _cpu_model(), "blas_threads": 1}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ---- GPU timing -----------------------------------------------------------------------

def step_distribution(fn, n):
    """Median, p10 and p90 of n individually timed calls (events around each call)."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in evs)
    pick = lambda f: t[min(n - 1, int(round(f * (n - 1))))]
    return {"n": n, "median_ms": pick(0.5), "p10_ms": pick(0.1), "p90_ms": pick(0.9)}


def time_calls(fn, steps, warmup):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


SWEEP_TC = (1, 2, 3, 5, 7)
SWEEP_TO = (0, 1, 2, 3)
SWEEP_LATENT = {3: "21x30x52", 2: "21x20x30"}


def sweep(args):
    """(Tc, To) grid of the ablation at two latents, causal, bf16 in / fp32 out."""
    import torch
    import synthetic as syn
    import hybrid_softmax_linear_amd as hs
    from hybrid_softmax_linear_amd import torch_api as ta
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    for ci in (3, 2):
        cfg = syn.config(ci)
        inp = syn.make_inputs(cfg)
        q, k, v, W = (inp[n].to(dev) for n in ("q", "k", "v", "W"))
        y = torch.empty(q.shape, dtype=torch.float32, device=dev)
        base = dict(B=cfg.B, H=cfg.H, T=cfg.T, HW=cfg.HW, D=cfg.D, F=cfg.F, dtype=hs.BF16,
                    y_dtype=hs.F32)
        full = hs.Desc(**base, Tc=cfg.T, To=0, mode=hs.CAUSAL)
        wsf = ta.workspace(hs.rehyat_hybrid_fwd_workspace(full), dev)
        full_ms = time_calls(lambda: hs.rehyat_hybrid_fwd(full, q, k, v, W, W, y, wsf, stream=stream),
                             max(3, args.steps // 4), 2)
        full_flop = 4 * cfg.D * cfg.N * cfg.N * cfg.B * cfg.H
        del wsf
        for Tc in SWEEP_TC:
            for To in SWEEP_TO:
                d = hs.Desc(**base, Tc=Tc, To=To, mode=hs.CAUSAL)
                ws = ta.workspace(hs.rehyat_hybrid_fwd_workspace(d), dev)
                ms = time_calls(lambda: hs.rehyat_hybrid_fwd(d, q, k, v, W, W, y, ws, stream=stream),
                                args.steps, args.warmup)
                flop = flop_model(cfg.B, cfg.H, cfg.T, cfg.HW, cfg.D, cfg.F, Tc, To, causal=True)[0]
                print(json.dumps({
                    "sweep": SWEEP_LATENT[ci], "B": cfg.B, "H": cfg.H,
                    "Tc": Tc, "To": To, "ms": ms, "tokens_per_s": cfg.B * cfg.N / (ms * 1e-3),
                    "tflops": flop / (ms * 1e-3) / 1e12, "flop": flop,
                    "full_softmax_ms": full_ms, "full_over_hybrid_flop": full_flop / flop,
                    "full_over_hybrid_time": full_ms / ms}), flush=True)
                del ws
        del q, k, v, W, y
    return 0


MLP_HIDDEN = 128   # hidden units of the learned feature map in the timed configurations


def feature_map_setup(kind, cfg, dev):
    """(Desc fields, Wq, Wk, phi FLOPs per row, label) of a feature map: "poly2" (the fixed
    map with the workload's W), "elu" (1 + elu) or "mlp" (the learned polynomial map with
    MLP_HIDDEN hidden units, P = 2, seeded parameters)."""
    import synthetic as syn
    import hybrid_softmax_linear_amd as hs
    from hybrid_softmax_linear_amd import torch_api as ta
    if kind == "elu":
        return dict(F=cfg.D, phi_kind=hs.PHI_ELU), None, None, 0, "1 + elu (F = D)"
    if kind == "mlp":
        h = MLP_HIDDEN
        pq = syn.make_mlp_map_params(cfg.D, h, cfg.F, seed=cfg.seed + 101)
        pk = syn.make_mlp_map_params(cfg.D, h, cfg.F, seed=cfg.seed + 102)
        bq = ta.mlp_param_block(pq["W1"], pq["b1"], pq["W2"], pq["b2"]).to(dev)
        bk = ta.mlp_param_block(pk["W1"], pk["b1"], pk["W2"], pk["b2"]).to(dev)
        return (dict(F=cfg.F, phi_kind=hs.PHI_MLP, phi_hidden=h, phi_parts=2), bq, bk,
                2 * cfg.D * h + 2 * h * cfg.F, f"learned polynomial map (h {h}, P 2)")
    return dict(F=cfg.F), None, None, 2 * cfg.D * cfg.F, "fixed map 1 + u + u^2/2"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the default line: time every (Tc, To) of the pages' "
                         "ablation grid at the 21x30x52 and 21x20x30 latents next to full "
                         "softmax, one JSON line per configuration")
    ap.add_argument("--stream", action="store_true",
                    help="27 recurrent steps over the 81x30x52 latent per step")
    ap.add_argument("--bwd", action="store_true",
                    help="instead of the default line: the backward of the causal form "
                         "(rehyat_hybrid_bwd) on the same workload")
    ap.add_argument("--workload", choices=("c3", "c2", "c5"), default="c3",
                    help="whole-sequence workload of the line: c3 the 21x30x52 causal latent "
                         "(the metric's, default), c2 the 21x20x30 bidirectional latent "
                         "(320x480, B1), c5 the 49x30x52 wide-chunk latent (Tc 7, To 3, F 256)")
    ap.add_argument("--phi", choices=("poly2", "elu", "mlp"), default="poly2",
                    help="feature map of the timed step (default: the fixed map)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy (reference kernel for "
                         "the FETCH_SIZE / WRITE_SIZE counter scale)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus "
              f"{args.gpus}); per-GPU throughput is the value at --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import synthetic as syn
    import hybrid_softmax_linear_amd as hs
    from hybrid_softmax_linear_amd import torch_api as ta

    hs.lib()   # fail loudly if the HIP library is missing
    if args.sweep:
        return sweep(args)
    if args.bwd:
        return bench_bwd(args)
    if args.stream:
        return bench_stream(args)
    cfg = syn.config(int(args.workload[1]))
    headline = args.workload == "c3"
    causal = cfg.mode == "causal"
    inp = syn.make_inputs(cfg)
    cpu = None if (args.no_cpu_baseline or not headline) else cpu_baseline(inp, cfg)
    print(f"# cpu baseline done: {cpu and round(cpu['value'], 1)} tokens/s", file=sys.stderr,
          flush=True)

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    q, k, v, W = (inp[n].to(dev) for n in ("q", "k", "v", "W"))
    base = dict(B=cfg.B, H=cfg.H, T=cfg.T, HW=cfg.HW, D=cfg.D, Tc=cfg.Tc, To=cfg.To,
                dtype=hs.BF16, y_dtype=hs.F32, mode=hs.CAUSAL if causal else hs.BIDIR)
    fields, Wq, Wk, phi_flop, phi_label = feature_map_setup(args.phi, cfg, dev)
    Wq = W if Wq is None and args.phi == "poly2" else Wq
    Wk = W if Wk is None and args.phi == "poly2" else Wk
    desc = hs.Desc(**base, **fields)
    ws = ta.workspace(hs.rehyat_hybrid_fwd_workspace(desc), dev)
    y = torch.empty(q.shape, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    def step():
        hs.rehyat_hybrid_fwd(desc, q, k, v, Wq, Wk, y, ws, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    hs.rehyat_timing_enable(True)
    ms = time_calls(step, args.steps, 0)
    kern_ms, launches = hs.rehyat_timing_read()
    hs.rehyat_timing_enable(False)
    kern_avg = kern_ms / max(launches, 1)
    # after the timed region: the spread of single steps
    dist = step_distribution(step, 50)

    total_flop, attn_flop, state_flop, pairs = flop_model(cfg.B, cfg.H, cfg.T, cfg.HW, cfg.D,
                                                          desc.F, cfg.Tc, cfg.To, causal=causal,
                                                          phi_row_flop=phi_flop)
    tokens = cfg.B * cfg.N
    tflops = total_flop / (ms * 1e-3) / 1e12
    attn_tflops = attn_flop / (kern_avg * 1e-3) / 1e12
    print(f"# step {ms:.3f} ms, attention kernel {kern_avg:.3f} ms ({launches} launches)",
          file=sys.stderr, flush=True)

    context = {}
    if not args.no_context and args.phi == "poly2" and headline:
        # the other feature maps of key design 3, same workload
        for kind in ("mlp", "elu"):
            f2, wq2, wk2, pf2, _ = feature_map_setup(kind, cfg, dev)
            d2 = hs.Desc(**base, **f2)
            ws2 = ta.workspace(hs.rehyat_hybrid_fwd_workspace(d2), dev)
            ms2 = time_calls(lambda: hs.rehyat_hybrid_fwd(d2, q, k, v, wq2, wk2, y, ws2,
                                                           stream=stream),
                             max(3, args.steps // 2), 2)
            fl2 = flop_model(cfg.B, cfg.H, cfg.T, cfg.HW, cfg.D, d2.F, cfg.Tc, cfg.To,
                             causal=True, phi_row_flop=pf2)[0]
            name = "learned_map" if kind == "mlp" else "elu_map"
            context[f"{name}_ms"] = ms2
            context[f"{name}_tokens_per_s"] = tokens / (ms2 * 1e-3)
            context[f"{name}_tflops"] = fl2 / (ms2 * 1e-3) / 1e12
            del ws2, wq2, wk2
    if not args.no_context and args.phi == "poly2" and headline:
        # the same causal computation as 7 recurrent steps (chunks resident, contiguous)
        Np = cfg.Tc * cfg.HW
        chunks = [tuple(x[:, :, t * Np:(t + 1) * Np].contiguous() for x in (q, k, v))
                  for t in range(cfg.n_chunks)]
        rec = ta.Recurrent(cfg.B, cfg.H, cfg.D, cfg.F, T=cfg.T, HW=cfg.HW, Tc=cfg.Tc, To=cfg.To,
                           device=dev)
        yc = torch.empty(chunks[0][0].shape, dtype=torch.float32, device=dev)

        def rec_pass():
            rec.t = 0
            for (qc, kc, vc) in chunks:
                rec.step(qc, kc, vc, W, out=yc)

        rec_ms = time_calls(rec_pass, max(3, args.steps // 2), 2)
        context["recurrent_7_steps_ms"] = rec_ms
        context["recurrent_tokens_per_s"] = tokens / (rec_ms * 1e-3)
        del chunks, rec, yc
        # bidirectional chunked form, same shape
        dbi = hs.Desc(**{**desc.__dict__, "mode": hs.BIDIR})
        wsb = ta.workspace(hs.rehyat_hybrid_fwd_workspace(dbi), dev)
        bi_ms = time_calls(lambda: hs.rehyat_hybrid_fwd(dbi, q, k, v, W, W, y, wsb, stream=stream),
                           max(3, args.steps // 2), 2)
        bi_flop = flop_model(cfg.B, cfg.H, cfg.T, cfg.HW, cfg.D, cfg.F, cfg.Tc, cfg.To, causal=False)[0]
        context["bidir_ms"] = bi_ms
        context["bidir_tflops"] = bi_flop / (bi_ms * 1e-3) / 1e12
        del wsb
        # full softmax attention of the same shape: one chunk spanning all 21 frames
        dfull = hs.Desc(**{**desc.__dict__, "Tc": cfg.T, "To": 0})
        wsf = ta.workspace(hs.rehyat_hybrid_fwd_workspace(dfull), dev)
        full_flop = 4 * cfg.D * cfg.N * cfg.N * cfg.B * cfg.H
        full_ms = time_calls(lambda: hs.rehyat_hybrid_fwd(dfull, q, k, v, W, W, y, wsf,
                                                           stream=stream), 3, 1)
        context["full_softmax_ms"] = full_ms
        context["full_softmax_tflops"] = full_flop / (full_ms * 1e-3) / 1e12
        context["full_over_hybrid_time"] = full_ms / ms
        del wsf
        try:
            qs, ks_, vs = q, k, v
            sdpa = lambda: torch.nn.functional.scaled_dot_product_attention(qs, ks_, vs)
            sd_ms = time_calls(sdpa, 3, 1)
            context["torch_sdpa_full_softmax_ms"] = sd_ms
            context["torch_sdpa_full_softmax_tflops"] = full_flop / (sd_ms * 1e-3) / 1e12
        except Exception as e:  # third-party context only
            context["torch_sdpa_error"] = str(e)[:200]

    if headline:
        metric = METRIC
        workload = (f"21x30x52 latent (480x832, 5 s): B2 H12 D128 F{desc.F}, Tc3 To1, causal, "
                    f"one rehyat_hybrid_fwd call per step"
                    + ("" if args.phi == "poly2" else f", {phi_label}"))
    else:
        lat = f"{cfg.T}x{cfg.HW // (52 if cfg.HW == 1560 else 30)}x{52 if cfg.HW == 1560 else 30}"
        form = "causal" if causal else "bidirectional"
        metric = f"hybrid-attn tokens/s & TFLOP/s per MI355X at {lat.replace('x', '×')} ({form}), % of MFMA peak"
        workload = (f"{lat} latent: B{cfg.B} H{cfg.H} D{cfg.D} F{desc.F}, Tc{cfg.Tc} To{cfg.To}, "
                    f"{form}, one rehyat_hybrid_fwd call per step"
                    + ("" if args.phi == "poly2" else f", {phi_label}"))
    result = {
        "metric": metric,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": workload,
                   "global_batch": cfg.B, "seq_len": cfg.N, "parallelism": "none (1 GPU)",
                   "y_dtype": "fp32"},
        "tflops": tflops,
        "mfma_peak_frac": tflops / MFMA_PEAK_BF16_TFLOPS,
        "flop_per_step": total_flop,
        "step_ms_distribution": dist,
        "roofline": {"bound": "mfma", "kernel": attn_kernel_name(cfg, desc.F),
                     "achieved": attn_tflops, "peak": MFMA_PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / MFMA_PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic() if headline and args.phi == "poly2" else None,
                     "flop_per_launch": attn_flop, "avg_launch_ms": kern_avg,
                     "launches_timed": launches},
        "cpu_baseline": cpu,
        "context": context,
    }
    print(json.dumps(result))
    return 0


if __name__ == "__main__":
    sys.exit(main())
