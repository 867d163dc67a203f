"""Benchmark of the strip-wise linear cross-entropy on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is the whole path on one batch: lce_forward (every strip folded into
the running per-token state, then finalised) and lce_backward (every strip
recomputed, its gradient strip formed, dH and dW accumulated), with inputs
already resident in HBM.  The metric is the fused fwd+bwd rate 8*N*H*V / time
in TFLOP/s, on the 131072-token workload (H=2048, V=151936, strip 8192, bf16)
unless --workload says otherwise.

Printed on one JSON line: the metric, the per-kernel roofline of the kernel
that takes most of the time (its algorithmic FLOP per launch over its
average launch time, measured with HIP events on the library's stream), and
the CPU oracle timed on a bounded sample of the same workload on the host
cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused linear-CE fwd+bwd TFLOP/s (8·N·H·V) and % bf16 MFMA peak"
DEFAULT_WORKLOAD = "bf16_n128k_h2k_v152k"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # MI355X published dense MFMA peaks
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--strip", type=int, default=0,
                    help="strip width Vs instead of the workload's (natural fold order only)")
    ap.add_argument("--backward", default="strip", choices=["strip", "one_sweep", "two_sweeps"],
                    help="backward form: the strip path (lce_backward), or the backward "
                         "without a strip buffer (lce_backward_fused) in one or two sweeps")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="tokens of the workload the CPU oracle is timed on")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the per-kernel timing pass")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (HBM counter scale)")
    return ap.parse_args()


def ensure_built():
    from vocab_projection_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from vocab_projection_amd import build
        build.build()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested).", file=sys.stderr)
        sys.exit(2)

    ensure_built()
    import torch
    from vocab_projection_amd import binding as B
    from vocab_projection_amd import synthetic as S

    w = S.WORKLOADS.get(args.workload) or S.EXTRA_WORKLOADS[args.workload]
    if args.strip:
        if w.shards:
            print("--strip applies to workloads folded in natural order", file=sys.stderr)
            sys.exit(2)
        # another configuration: its own name, so no stored counter summary applies
        w = w.with_(strip=args.strip, name=f"{w.name}_strip{args.strip}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    t0 = time.time()
    hid_np = S.hidden(w, threads=16)
    w_np = S.weight(w, threads=16)
    t_np = S.targets(w)
    h = torch.from_numpy(hid_np).to(dev).to(dt)
    W = torch.from_numpy(w_np).to(dev).to(dt)
    t = torch.from_numpy(t_np).to(dev)
    log(f"inputs {w.name}: {time.time() - t0:.1f}s")

    p = B.make_problem(h, W, ignore_index=S.IGNORE_INDEX, reduction=w.reduction, strip=w.strip)
    order = S.fold_order(w)
    natural = w.shards == 0
    ws = B.workspace(p, dev)
    fused = args.backward != "strip"
    if fused:
        if not natural:
            print("--backward applies to workloads folded in natural order", file=sys.stderr)
            sys.exit(2)
        fmode = B.FUSED_MODES[args.backward]
        fws = torch.empty(B.lce_backward_fused_workspace_bytes(p, fmode), dtype=torch.uint8,
                          device=dev)
        args.no_breakdown = True
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    lse = torch.empty(w.n_tokens, dtype=torch.float32, device=dev)
    dh = torch.empty(h.shape, dtype=torch.float32, device=dev)
    dw = torch.empty(W.shape, dtype=torch.float32, device=dev)
    go = torch.tensor([w.grad_out], dtype=torch.float32, device=dev)

    def step():
        if fused:
            B.lce_forward(p, h, W, t, loss, lse, None, ws)
            B.lce_backward_fused(p, h, W, t, lse, go, dh, dw, fmode, fws)
        elif natural:
            B.lce_forward(p, h, W, t, loss, lse, None, ws)
            B.lce_backward(p, h, W, t, lse, go, dh, dw, ws)
        else:
            B.lce_forward_begin(p, ws)
            for v0, vl in order:
                B.lce_forward_fold(p, h, W[v0:v0 + vl], v0, vl, t, ws)
            B.lce_forward_end(p, t, loss, lse, None, ws)
            B.lce_backward_begin(p, t, go, ws)
            for k, (v0, vl) in enumerate(order):
                B.lce_backward_fold(p, h, W[v0:v0 + vl], v0, vl, t, lse, dh, k > 0,
                                    dw[v0:v0 + vl], ws)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} loss={loss.item():.6f}")

    # memory: nothing beyond the caller's buffers may be allocated by a step
    free_before = torch.cuda.mem_get_info(dev)[0]
    torch.cuda.reset_peak_memory_stats(dev)
    alloc_before = torch.cuda.memory_allocated(dev)

    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / args.steps
    log(f"timed {args.steps} steps: {ms_per_step:.2f} ms/step (wall {wall:.2f}s)")
    peak_alloc_extra = torch.cuda.max_memory_allocated(dev) - alloc_before
    free_after = torch.cuda.mem_get_info(dev)[0]

    tflops = w.flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "n_tokens": w.n_tokens, "hidden": w.hidden,
                   "vocab": w.vocab, "strip": w.strip, "reduction": w.reduction,
                   "fold_order": "natural" if natural else f"ring of {w.shards} shards",
                   "backward": args.backward},
        "pct_of_peak": round(100.0 * tflops / peak, 2),
        "memory": {
            "workspace_bytes": B.lce_workspace_bytes(p),
            "backward_workspace_bytes": fws.numel() if fused else B.lce_workspace_bytes(p),
            "strip_bytes": w.n_tokens * w.strip * w.elt_bytes,
            "full_logits_bytes": w.n_tokens * w.vocab * w.elt_bytes,
            "allocator_peak_extra_bytes": int(peak_alloc_extra),
            "device_free_delta_bytes": int(free_before - free_after),
        },
    }

    if not args.no_breakdown:
        result["kernels"], result["roofline"] = kernel_breakdown(
            args, B, torch, w, p, h, W, t, lse, dh, dw, go, ws, order, loss, peak)

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = n

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, hid_np, w_np, t_np, args.cpu_rows)
    print(json.dumps(result), flush=True)


KERNEL_SOURCES = ("tile_engine.h", "tile_engine_w4.h", "lce_kernels.hip", "lce_kernels.h")


def kernel_source_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "vocab_projection_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, step: str):
    """Bytes per launch of `step` that leave the L2 caches towards memory, from
    the committed FETCH_SIZE / WRITE_SIZE summary (scaled by the copy-kernel
    calibration; MALL hits included, since no counter on this part separates
    them from HBM), or None when there is none for this workload or the
    kernels changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        prof = json.load(f)
    if prof.get("source_sha256") != kernel_source_sha256():
        return None
    k = prof.get("kernels", {}).get(step)
    return None if k is None else k["l2_egress_bytes_per_dispatch"]


def kernel_breakdown(args, B, torch, w, p, h, W, t, lse, dh, dw, go, ws, order, loss, peak):
    """Run the timed step's launches again, one call per kernel, with an event
    pair around each on the stream the library launches on; return per-kernel
    times and the roofline of the kernel with the largest total time.

    The launches are those of the timed step: in natural order the forward
    folds as lce_forward does (ranges of lce_forward_fold_max rows, so one
    strip_lse launch over the whole vocabulary when it fits), and each strip of
    the backward runs strip_grad, then dH and dW as two launches or as the one
    shared launch that lce_backward_fold makes for that strip."""
    # bf16 GEMMs run on the one-wave-per-SIMD engine from K >= 768 (the strip
    # kernels, K = H) or K >= 1024 (dH, K = strip rows; dW, K = tokens; the
    # shared dH + dW launch)
    bf16 = w.dtype == "bf16"
    w4 = "_w4" if bf16 and w.hidden >= 768 else f"<{'bf16' if bf16 else 'float'}>"
    w4_dw = "_w4" if bf16 and w.n_tokens >= 1024 else ""
    w4_dh = "_w4" if bf16 and min(w.strip or w.vocab, w.vocab) >= 1024 else ""
    kernels = {
        "strip_lse": "lce::strip_lse_kernel" + w4,
        "merge": "lce::fold_kernel",
        "strip_grad": "lce::strip_grad_kernel" + w4,
        "gemm_dh": f"lce::gemm_f32out_kernel{w4_dh}<A K-contig, B MN-contig>",
        "gemm_dw": f"lce::gemm_f32out_kernel{w4_dw}<A MN-contig, B MN-contig>",
        "gemm_dh_dw": f"lce::gemm_dh_dw_kernel{w4_dw} (dH and dW sharing one launch)",
    }
    # algorithmic FLOP per (token x vocabulary row) of each launch
    flops_per_elem = {"strip_lse": 2.0 * w.hidden, "strip_grad": 2.0 * w.hidden,
                      "gemm_dh": 2.0 * w.hidden, "gemm_dw": 2.0 * w.hidden,
                      "gemm_dh_dw": 4.0 * w.hidden}
    recs = {k: [] for k in kernels}

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    if w.shards:
        fwd_ranges = order
    else:
        wide = B.lce_forward_fold_max(p)
        fwd_ranges = [(v0, min(wide, w.vocab - v0)) for v0 in range(0, w.vocab, wide)]
    launches = {vl: B.lce_backward_fold_gemm_launches(p, vl) for _, vl in order}
    S_STRIP, S_MERGE = B.LCE_STEP_STRIP, B.LCE_STEP_MERGE
    S_GRAD, S_DH, S_DW = B.LCE_STEP_GRAD, B.LCE_STEP_DHIDDEN, B.LCE_STEP_DWEIGHT
    for _ in range(args.steps):
        B.lce_forward_begin(p, ws)
        for v0, vl in fwd_ranges:
            for k, st in (("strip_lse", S_STRIP), ("merge", S_MERGE)):
                a = ev()
                B.lce_forward_fold_steps(p, h, W[v0:v0 + vl], v0, vl, t, ws, st)
                recs[k].append((a, ev(), vl))
        B.lce_forward_end(p, t, loss, lse, None, ws)
        B.lce_backward_begin(p, t, go, ws)
        for i, (v0, vl) in enumerate(order):
            parts = [("strip_grad", S_GRAD)]
            parts += [("gemm_dh", S_DH), ("gemm_dw", S_DW)] if launches[vl] == 2 \
                else [("gemm_dh_dw", S_DH | S_DW)]
            for k, st in parts:
                a = ev()
                B.lce_backward_fold_steps(p, h, W[v0:v0 + vl], v0, vl, t, lse, dh, i > 0,
                                          dw[v0:v0 + vl], ws, st)
                recs[k].append((a, ev(), vl))
    torch.cuda.synchronize()
    out = {}
    for k, lst in recs.items():
        if not lst:
            continue
        ms = [a.elapsed_time(b) for a, b, _ in lst]
        entry = {"kernel": kernels[k], "launches_per_step": len(ms) // args.steps,
                 "avg_ms": round(float(np.mean(ms)), 4),
                 "total_ms_per_step": round(float(np.sum(ms)) / args.steps, 3)}
        if k in flops_per_elem:
            fl = sum(flops_per_elem[k] * w.n_tokens * vl for _, _, vl in lst)
            entry["tflops"] = round(fl / (np.sum(ms) * 1e-3) / 1e12, 2)
            entry["algorithmic_flop_per_launch"] = fl / len(ms)
        out[k] = entry
    dom = max((k for k in flops_per_elem if k in out), key=lambda k: out[k]["total_ms_per_step"])
    achieved = out[dom]["tflops"]
    roof = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": measured_traffic(w.name, dom),
            "traffic_counts": "bytes leaving L2 per launch (FETCH_SIZE + WRITE_SIZE, calibrated "
                              "on a 1 GiB copy); MALL hits included",
            "kernel": out[dom]["kernel"],
            "step": dom, "avg_launch_ms": out[dom]["avg_ms"],
            "algorithmic_flop_per_launch": out[dom]["algorithmic_flop_per_launch"]}
    log("per-kernel:", json.dumps(out))
    return out, roof


def cpu_facts():
    """CPU model, logical CPUs, physical cores (distinct package/core pairs) and
    the CPUs this process may run on."""
    model, pairs = None, set()
    phys = core = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k, v = k.strip(), v.strip()
                if k == "model name" and model is None:
                    model = v
                elif k == "physical id":
                    phys = v
                elif k == "core id":
                    core = v
                elif not k and phys is not None and core is not None:
                    pairs.add((phys, core))
                    phys = core = None
        if phys is not None and core is not None:
            pairs.add((phys, core))
    except OSError:
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count(),
            "physical_cores": len(pairs) or None,
            "affinity_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(w, hid_np, wt, t_np, rows):
    """The CPU oracle, as it is, on the first `rows` tokens with the full weight,
    on every thread of the host's BLAS pool; plus its single-thread rate on the
    256-token float32 workload (whole problem), and the full workload's time
    projected from the measured rate (labelled as a projection)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import lce_oracle as O
    from vocab_projection_amd import synthetic as S

    hs, ts = hid_np[:rows], t_np[:rows]
    t0 = time.perf_counter()
    O.forward(hs, wt, ts, ignore_index=S.IGNORE_INDEX, reduction=w.reduction)
    O.backward(hs, wt, ts, ignore_index=S.IGNORE_INDEX, reduction=w.reduction,
               grad_out=w.grad_out)
    sec = time.perf_counter() - t0
    flops = 8.0 * rows * w.hidden * w.vocab
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    rate = flops / sec

    tiny = S.WORKLOADS["tiny_f32"]
    th, tw, tt = S.hidden(tiny), S.weight(tiny), S.targets(tiny)
    with threadpool_limits(limits=1):
        reps, t1 = 0, time.perf_counter()
        while reps < 3 or time.perf_counter() - t1 < 1.0:
            O.forward(th, tw, tt, ignore_index=S.IGNORE_INDEX, reduction=tiny.reduction)
            O.backward(th, tw, tt, ignore_index=S.IGNORE_INDEX, reduction=tiny.reduction)
            reps += 1
        st_sec = (time.perf_counter() - t1) / reps
    out = {"value": round(rate / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads),
           "kind": "oracle", "seconds": round(sec, 2),
           "sample": f"first {rows} of {w.n_tokens} tokens with the full weight "
                     f"(H={w.hidden}, V={w.vocab}): oracle forward + backward in float64, "
                     f"8*{rows}*H*V FLOP, on {threads} BLAS threads",
           "single_thread": {"value": round(tiny.flops / st_sec / 1e12, 5), "unit": "TFLOP/s",
                             "sample": f"{tiny.name} whole (N={tiny.n_tokens}, H={tiny.hidden}, "
                                       f"V={tiny.vocab}, float32 inputs), oracle forward + "
                                       f"backward, 1 thread, {reps} runs",
                             "seconds_per_run": round(st_sec, 4)},
           "projected_full_workload_seconds": round(w.flops / rate, 1),
           "projection": f"8*N*H*V of the whole workload ({w.flops:.4g} FLOP) over the "
                         f"measured {threads}-thread rate; not measured"}
    out.update(cpu_facts())
    return out


if __name__ == "__main__":
    main()
