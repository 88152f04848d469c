#!/usr/bin/env python3
"""Benchmark of the VDA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 768p_bf16] [--gated]

One step = one whole forward pass (statistics, scans, readout) over one batch of
seeded synthetic input already resident in HBM.  Prints ONE JSON line with the
headline metric (video tokens/s at the 768p shape), the HBM roofline of the
dominant kernel (timed live with HIP events on the launch stream) and the float64
oracle's throughput on a bounded sample of the same workload on the host cores.

Profiling helpers (used to produce the committed summaries under profiles/):
    python bench.py --copy-probe            plain copy kernel of known size, for
                                            calibrating rocprofv3 byte counters
    python bench.py --summarize-stats CSV   kernel_stats.csv -> text summary
    python bench.py --summarize-pmc FETCH_CSV WRITE_CSV COPY_FETCH_CSV COPY_WRITE_CSV
    python bench.py --summarize-counters CSV  any counter pass -> per-kernel averages

With the CPU leg on (the default), the output of the last timed pass is also compared with
the oracle on every (b,h) slice the CPU leg computes ("parity" in the JSON line).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}  # dense MFMA, vendor figures
KERNEL_SOURCES = {"stats": "stats.hip", "scan": "scan.hip", "readout": "readout.hip"}
# kernels of each forward stage (the chunked scan is three launches: local pass, carry, rerun)
KERNEL_SYMBOLS = {"stats": ("stats_bf16_kernel",), "scan": ("scan_bf16_kernel", "chunk_carry_kernel"),
                  "readout": ("readout_bf16_kernel",)}
GATED_READOUT_SYMBOL = "readout_gated_kernel"  # the readout with the gated epilogue (--gated)
COPY_PROBE_BYTES = 1 << 30


def source_hash(kernel: str) -> str:
    path = os.path.join(ROOT, "frame_wise_delta_vda_amd", "csrc", KERNEL_SOURCES[kernel])
    h = hashlib.sha256()
    for p in (path, os.path.join(ROOT, "frame_wise_delta_vda_amd", "csrc", "vda_device.h")):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic(w, gated=False):
    """Bytes and flops the method itself requires, per launch of each stage.  With the gated
    epilogue the readout also reads the per-head weights and computes the two projections
    (O W_g^T and O W_o^T, dv x dv per token) on top of O = Q W."""
    es, eo = w.elem_bytes, w.out_bytes  # input and output element bytes
    BH = w.B * w.H
    tok = BH * (w.F * w.n + w.T)
    vid = BH * w.F * w.n
    readout = {"bytes": vid * (w.d * es + w.dv * eo), "flops": vid * 2 * w.d * w.dv}
    if gated:
        readout = {"bytes": readout["bytes"] + w.H * (2 * w.dv * w.dv * 2 + w.dv * 4),
                   "flops": readout["flops"] + vid * 2 * 2 * w.dv * w.dv}
    return {
        "stats": {"bytes": tok * (w.d + w.dv) * es,
                  "flops": tok * (2 * w.d * w.d + 2 * w.d * w.dv) + BH * (w.F + 1) * 2 * w.d ** 3},
        "scan": {"bytes": 0, "flops": 2 * BH * (w.F + 1) * 2 * w.d * w.d * w.dv},
        "readout": readout,
    }


def read_traffic(workload_name):
    """Per-launch HBM bytes from the committed counter summary, or None per kernel when
    the summary is missing or the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload_name}.txt")
    out = {}
    if not os.path.exists(path):
        return out
    with open(path) as f:
        for line in f:
            if line.startswith("traffic "):
                parts = dict(kv.split("=", 1) for kv in line.split()[1:])
                k = parts["kernel"]
                if parts.get("source") == source_hash(k):
                    out[k] = float(parts["bytes_per_launch"])
    return out


def host_cpu():
    """(model name, usable cores, BLAS threads to use) of the host this runs on.  The cores are
    the affinity mask's; where the environment caps the thread count (OMP_NUM_THREADS, set to
    the per-GPU CPU share on shared boxes) the BLAS pool takes the smaller of the two."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(cores, int(cap)) if cap.isdigit() and int(cap) > 0 else cores
    return model, cores, threads


def cpu_baseline(w, arrays, budget_s=20.0, max_heads=None, gate=None, gpu_out=None):
    """Time the float64 oracle on whole (b,h) slices of the same inputs until ~budget_s
    (with the gated epilogue when gate holds the weights as float64).  When gpu_out (the
    timed GPU output, on the host) is given, every slice the oracle computed is also compared
    with it: the max per-(b,h,frame) relative Frobenius error is returned with the baseline."""
    import numpy as np
    import threadpoolctl
    import oracle
    import workloads as W

    model, cores, threads = host_cpu()
    heads = [(b, h) for b in range(w.B) for h in range(w.H)][: max_heads or None]
    spent, done, worst = 0.0, 0, 0.0
    with threadpoolctl.threadpool_limits(limits=threads, user_api="blas"):
        for b, h in heads:
            x = {k: W.storage_to_float64(w, arrays[k][b, h]) for k in W.TENSORS}
            t0 = time.perf_counter()
            if gate is None:
                ref = oracle.vda_forward_head(x["q"], x["k"], x["v"], x["text_k"], x["text_v"], w.lam)
            else:
                ref = oracle.vda_forward_gated_head(x["q"], x["k"], x["v"], x["text_k"], x["text_v"], w.lam,
                                                    gate["w_gate"][h], gate["b_gate"][h], gate["w_out"][h])
            spent += time.perf_counter() - t0
            done += 1
            if gpu_out is not None:
                got = gpu_out[b, h].float().numpy().astype(np.float64)
                diff = np.sqrt(np.sum((got - ref) ** 2, axis=(-2, -1)))
                nrm = np.maximum(np.sqrt(np.sum(ref ** 2, axis=(-2, -1))), 1e-300)
                worst = max(worst, float(np.max(diff / nrm)))
            del x, ref
            if spent >= budget_s:
                break
    toks = done * w.F * w.n
    res = {"value": toks / spent, "unit": "video tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{done} of {w.B * w.H} (b,h) slices of {w.name} ({toks} video tokens), "
                     f"numpy float64, {spent:.1f} s",
           "cpu_model": model, "host_cores": cores, "blas_threads": threads}
    parity = None
    if gpu_out is not None:
        parity = {"max_rel_err": worst, "heads": done, "of_heads": w.B * w.H,
                  "tol": 1e-4 if w.dtype == "f32" else 1e-2,
                  "metric": "max over (b,h,frame) of ||O_gpu - O_oracle||_F / ||O_oracle||_F"}
    return res, parity


# Arithmetic of each stage, per input type (the contraction types the kernels use).
ARITHMETIC = {
    "f32": {"stats": "fp32 MFMA", "scan": "fp32 MFMA", "readout": "fp32 MFMA"},
    "bf16": {"stats": "bf16 MFMA, fp32 accumulate; fp32 inverse", "scan": "split-bf16 MFMA (fp32 chain)",
             "readout": "bf16 MFMA, fp32 accumulate"},
    "fp8": {"stats": "fp8 e4m3 MFMA at d = dv = 128 (bf16 MFMA at other widths), fp32 accumulate; fp32 inverse",
            "scan": "split-bf16 MFMA (fp32 chain)", "readout": "bf16 MFMA, fp32 accumulate"},
}


def to_device(w, arrays):
    import numpy as np
    import torch
    dev = {}
    for k, a in arrays.items():
        # bfloat16 as torch bfloat16, FP8 e4m3 codes as uint8, float32 as is
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16" \
            else torch.from_numpy(a)
        dev[k] = t.to("cuda")
    return dev


def run(args):
    import torch
    import workloads as W
    from frame_wise_delta_vda_amd import vda as binding

    w = W.by_name(args.workload)
    print(f"[bench] {w.name}: generating inputs", file=sys.stderr, flush=True)
    arrays = W.full_storage(w)
    dev = to_device(w, arrays)
    if args.no_cpu_baseline:
        del arrays
    out = torch.empty(w.shapes()["out"], device="cuda",
                      dtype=torch.float32 if w.dtype == "f32" else torch.bfloat16)
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    if args.scan_chunk is not None:
        plan.set_scan_chunk(args.scan_chunk)
    scan_chunk = plan.scan_chunk if w.dtype != "f32" else 0
    q, k, v, tk, tv = (dev[x] for x in W.TENSORS)
    gate = None
    if args.gated:
        import numpy as np
        gate = W.gate_weights(w)
        bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        wg, wo = bits(gate["w_gate"]), bits(gate["w_out"])
        bg = torch.from_numpy(np.ascontiguousarray(gate["b_gate"])).cuda()

    def step():
        # one whole forward pass through the C ABI: the product call (statistics, scans and
        # readout, three launches on the current stream), with or without the gated epilogue
        if gate is None:
            plan.forward(q, k, v, tk, tv, out)
        else:
            plan.forward_gated(q, k, v, tk, tv, wg, bg, wo, out)

    print(f"[bench] {w.name}: warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    names = ["stats", "scan", "readout"]
    bits = {"stats": binding.VDA_STAGE_STATS, "scan": binding.VDA_STAGE_SCAN, "readout": binding.VDA_STAGE_READOUT}
    # per-stage breakdown, outside the timed region: K passes with every stage's kernel timed by
    # the library's HIP events (recorded by each launch itself, on the launch stream)
    plan.enable_timing(args.steps)
    for _ in range(args.steps):
        step()
    calls, st_ms, sc_ms, rd_ms = plan.timings()
    if calls != args.steps:
        raise RuntimeError(f"timed {calls} of {args.steps} passes")
    kern_ms = {"stats": st_ms, "scan": sc_ms, "readout": rd_ms}
    dom = max(("stats", "readout"), key=lambda n: kern_ms[n])
    # the timed region: K whole passes, with only the dominant kernel carrying its events (each
    # timed stage adds an event pair to a pass), for its live duration
    plan.set_timed_stages(bits[dom])
    plan.enable_timing(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    calls, *live = plan.timings()
    if calls != args.steps:
        raise RuntimeError(f"timed {calls} of {args.steps} passes")
    live_ms = dict(zip(names, live))[dom]
    print(f"[bench] {w.name}: {ms_step:.3f} ms/step; " +
          ", ".join(f"{n} {kern_ms[n]:.3f} ms" for n in names) + f"; {dom} in the timed passes {live_ms:.3f} ms",
          file=sys.stderr, flush=True)

    alg = algorithmic(w, args.gated)
    prof_name = w.name + ("_gated" if args.gated else "") + (f"_scan_chunk{args.scan_chunk}" if args.scan_chunk else "")
    traffic = read_traffic(prof_name)
    kernels = {}
    kern_ms[dom] = live_ms  # the dominant kernel: its duration in the timed passes themselves
    for n in names:
        ms = kern_ms[n]
        entry = {"ms": round(ms, 4), "timed": "live, in the timed passes" if n == dom else "breakdown passes"}
        if alg[n]["bytes"]:
            gbs = alg[n]["bytes"] / (ms * 1e-3) / 1e9
            entry.update({"alg_bytes": alg[n]["bytes"], "GB/s": round(gbs, 1),
                          "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
        entry["TFLOP/s"] = round(alg[n]["flops"] / (ms * 1e-3) / 1e12, 2)
        # MFMA fraction against the dense peak of the stage's contraction type
        peak = MFMA_PEAK_TFLOPS["fp8" if (n == "stats" and w.dtype == "fp8" and w.d == 128 and w.dv == 128)
                                else "f32" if w.dtype == "f32" else "bf16"]
        entry["mfma_frac"] = round(entry["TFLOP/s"] / peak, 4)
        entry["traffic"] = traffic.get(n)
        kernels[n] = entry
    ach = kernels[dom]["GB/s"]
    whole_gbs = w.algorithmic_bytes() / (ms_step * 1e-3) / 1e9
    roofline = {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic.get(dom),
                # the whole step (all three kernels and the gaps between them) against the same
                # peak: the algorithmic bytes of the pass over the wall clock per step
                "whole_step": {"achieved": round(whole_gbs, 1), "frac": round(whole_gbs / HBM_PEAK_GBS, 4),
                               "ms": round(ms_step, 4)}}
    value = w.video_tokens / (ms_step * 1e-3)
    result = {
        "metric": "VDA forward video tokens/s at 768p shape; % of HBM/MFMA roofline",
        "value": round(value, 1),
        "unit": "video tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # arithmetic type of the path: FP8 inputs contract on the FP8 MFMA in the statistics
        # (d = dv = 128) and are converted to bfloat16 for the readout
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8_e4m3+bf16"}[w.dtype],
        "data": "synthetic",
        "config": {"workload": w.name, "input_dtype": w.dtype, "arithmetic": ARITHMETIC[w.dtype],
                   "epilogue": "sigmoid gate and output projection per head" if args.gated else "none",
                   "scan": (f"chunked, {scan_chunk} frames per chunk ({-(-w.F // scan_chunk)} chunks)"
                            if scan_chunk else "serial"), "B": w.B, "H": w.H, "F": w.F, "n": w.n, "d": w.d, "dv": w.dv,
                   "T": w.T, "lambda": w.lam, "video_tokens_per_step": w.video_tokens,
                   "alg_bytes_per_step": w.algorithmic_bytes(),
                   "whole_step_GB/s": round(w.algorithmic_bytes() / (ms_step * 1e-3) / 1e9, 1)},
        "roofline": roofline,
        "kernels": kernels,
    }
    plan.close()
    out_host = None if args.no_cpu_baseline else out.cpu()  # the output of the last timed pass
    del dev, out
    if not args.no_cpu_baseline:
        print(f"[bench] {w.name}: timing the oracle on host cores", file=sys.stderr, flush=True)
        result["cpu_baseline"], result["parity"] = cpu_baseline(
            w, arrays, budget_s=args.cpu_budget, gate=W.gate_weights_float64(w, gate) if gate else None,
            gpu_out=out_host)
        print(f"[bench] {w.name}: parity against the oracle on {result['parity']['heads']} heads: "
              f"max rel err {result['parity']['max_rel_err']:.3e}", file=sys.stderr, flush=True)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def copy_probe(args):
    """A plain read-once/write-once elementwise kernel over COPY_PROBE_BYTES."""
    import torch
    n = COPY_PROBE_BYTES // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(max(args.steps, 1)):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": COPY_PROBE_BYTES, "copy_probe_bytes_written": COPY_PROBE_BYTES}))


def short_name(name: str) -> str:
    name = name.replace("(anonymous namespace)::", "").replace("void ", "", 1)
    return name.split("(")[0]


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def run_backward(args):
    """Time vda_backward (gradients of q, k, v and the text) after one forward pass on the same
    plan; one JSON line like the forward's, with the backward's own spans."""
    import numpy as np
    import torch
    import oracle
    import workloads as W
    from frame_wise_delta_vda_amd import vda as binding

    w = W.by_name(args.workload)
    if w.dtype != "bf16":
        raise SystemExit("the backward pass runs on bfloat16 workloads")
    print(f"[bench] backward {w.name}: generating inputs", file=sys.stderr, flush=True)
    arrays = W.full_storage(w)
    dev = to_device(w, arrays)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence((w.seed, 0xD0))))
    d_out_bits = W.float32_to_bf16_bits(rng.standard_normal(w.shapes()["out"], dtype=np.float32))
    d_out = torch.from_numpy(d_out_bits.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v, tk, tv = (dev[x] for x in W.TENSORS)
    plan = binding.Plan(w.B, w.H, w.F, w.n, w.d, w.dv, w.T, w.lam, w.dtype)
    out = torch.empty(w.shapes()["out"], device="cuda", dtype=torch.bfloat16)
    plan.forward(q, k, v, tk, tv, out)  # the statistics and states the backward pass reads
    grads = tuple(torch.empty_like(t) for t in (q, k, v, tk, tv))

    def step():
        plan.backward(q, k, v, tk, tv, d_out, grads=grads)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    plan.enable_timing(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    calls, st_ms, sc_ms, rd_ms = plan.timings()
    if calls != args.steps:
        raise RuntimeError(f"timed {calls} of {args.steps} passes")
    BH = w.B * w.H
    tok = BH * w.F * w.n
    ttok = BH * w.T
    e = 2  # bf16
    # bytes each span must move.  At d = dv = 128 the first span is the float32 state
    # recompute and one pass over (Q, dO) that forms dW = Q^T dO and dQ = dO W^T (reads Q, dO,
    # writes dQ); the products read K, V and write dK, dV (and the text's K, V in, gradients
    # out).  At other widths the first span is Q^T dO alone and dQ is one of the products.
    text = ttok * 2 * (w.d + w.dv) * e
    if w.d == 128 and w.dv == 128:
        first = "recompute_dw_dq"
        alg = {first: tok * (w.d + w.dv + w.d) * e, "products": tok * 2 * (w.d + w.dv) * e + text}
    else:
        first = "stats"
        alg = {first: tok * (w.d + w.dv) * e,
               "products": tok * (w.dv + w.d + w.dv + w.d + w.d + w.dv) * e + text}
    spans = {first: st_ms, "adjoint": sc_ms, "products": rd_ms}
    kernels = {n: {"ms": round(ms, 4)} for n, ms in spans.items()}
    for n in alg:
        gbs = alg[n] / (spans[n] * 1e-3) / 1e9
        kernels[n].update({"alg_bytes": alg[n], "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
    dom = max(alg, key=lambda n: spans[n])
    ach = kernels[dom]["GB/s"]
    # the whole backward must read Q, K, V, dO and write dQ, dK, dV (and the text's two pairs)
    whole = tok * (4 * w.d + 3 * w.dv) * e + ttok * 2 * (w.d + w.dv) * e
    result = {
        "metric": "VDA backward (gradients of q, k, v and text) video tokens/s at 768p shape; % of HBM roofline",
        "value": round(w.video_tokens / (ms_step * 1e-3), 1), "unit": "video tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "backward", "B": w.B, "H": w.H, "F": w.F, "n": w.n,
                   "d": w.d, "dv": w.dv, "T": w.T, "lambda": w.lam, "alg_bytes_per_step": whole,
                   "whole_step_GB/s": round(whole / (ms_step * 1e-3) / 1e9, 1)},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None},
        "kernels": kernels,
    }
    plan.close()
    if not args.no_cpu_baseline:
        print(f"[bench] backward {w.name}: timing the oracle on host cores", file=sys.stderr, flush=True)
        import threadpoolctl
        model, cores, threads = host_cpu()
        spent, done = 0.0, 0
        with threadpoolctl.threadpool_limits(limits=threads, user_api="blas"):
            for h in range(w.H):
                x = {kk: W.storage_to_float64(w, arrays[kk][0, h]) for kk in W.TENSORS}
                dO = W.bf16_bits_to_float32(d_out_bits[0, h]).astype(np.float64)
                t1 = time.perf_counter()
                oracle.vda_backward_head(x["q"], x["k"], x["v"], x["text_k"], x["text_v"], w.lam, dO)
                spent += time.perf_counter() - t1
                done += 1
                if spent >= args.cpu_budget:
                    break
        result["cpu_baseline"] = {"value": done * w.F * w.n / spent, "unit": "video tokens/s", "cores": threads,
                                  "kind": "oracle", "sample": f"{done} of {w.B * w.H} (b,h) slices of {w.name}, "
                                                              f"numpy float64 backward, {spent:.1f} s",
                                  "cpu_model": model, "host_cores": cores, "blas_threads": threads}
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def summarize_stats(args):
    rows = _rows(args.summarize_stats)
    print(f"# rocprofv3 --kernel-trace --stats summary")
    print(f"# command: {args.command}")
    print(f"{'kernel':<60} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}")
    for r in rows:
        name = r.get("Name") or r.get("KernelName") or r.get("Kernel_Name")
        short = short_name(name)[:60]
        print(f"{short:<60} {int(r['Calls']):>6} {float(r['AverageNs'])/1e3:>10.2f} "
              f"{float(r['MinNs'])/1e3:>10.2f} {float(r['MaxNs'])/1e3:>10.2f} {float(r['Percentage']):>6.2f}")


def _pmc_per_kernel(path, counter):
    """Average counter value per dispatch for each kernel in a counter_collection CSV."""
    acc = {}
    for r in _rows(path):
        if r.get("Counter_Name") != counter:
            continue
        name = r["Kernel_Name"]
        acc.setdefault(name, []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_pmc(args):
    """Per-launch HBM traffic of the VDA kernels from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by what the same counter reads for the copy probe."""
    import workloads as W
    fetch_csv, write_csv, cfetch_csv, cwrite_csv = args.summarize_pmc
    w = W.by_name(args.workload)
    prof_name = w.name + ("_gated" if args.gated else "") + (f"_scan_chunk{args.scan_chunk}" if args.scan_chunk else "")
    fetch = _pmc_per_kernel(fetch_csv, "FETCH_SIZE")
    write = _pmc_per_kernel(write_csv, "WRITE_SIZE")
    cf = _pmc_per_kernel(cfetch_csv, "FETCH_SIZE")
    cw = _pmc_per_kernel(cwrite_csv, "WRITE_SIZE")
    copy_name = max(cf, key=cf.get)
    f_scale = COPY_PROBE_BYTES / (cf[copy_name] * 1024.0)
    w_scale = COPY_PROBE_BYTES / (cw[copy_name] * 1024.0)
    alg = algorithmic(w, args.gated)
    print(f"# HBM traffic per launch, {prof_name}, from rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE")
    print(f"# command: {args.command}")
    print(f"# calibration: copy probe '{short_name(copy_name)[:50]}' over {COPY_PROBE_BYTES} B read + "
          f"{COPY_PROBE_BYTES} B written reads FETCH_SIZE {cf[copy_name]:.0f} KiB, WRITE_SIZE "
          f"{cw[copy_name]:.0f} KiB -> scale fetch x{f_scale:.4f}, write x{w_scale:.4f}")
    for kern, syms in KERNEL_SYMBOLS.items():
        if kern == "readout" and args.gated:
            syms = (GATED_READOUT_SYMBOL,)
        names = [n for n in fetch if any(sym in n for sym in syms)]
        if not names:
            continue
        # a stage's bytes per step: the per-dispatch averages of its kernels, summed
        fb = sum(fetch[n] for n in names) * 1024.0 * f_scale
        wb = sum(write.get(n, 0.0) for n in names) * 1024.0 * w_scale
        print(f"# {kern}: fetch {fb/1e9:.4f} GB, write {wb/1e9:.4f} GB per launch; algorithmic "
              f"{alg[kern]['bytes']/1e9:.4f} GB" + (f"; kernels: {', '.join(short_name(n) for n in names)}"
                                                    if len(names) > 1 else ""))
        print(f"traffic kernel={kern} bytes_per_launch={fb + wb:.0f} fetch_bytes={fb:.0f} "
              f"write_bytes={wb:.0f} alg_bytes={alg[kern]['bytes']} source={source_hash(kern)}")


def summarize_counters(args):
    """Per-dispatch averages of every counter in a rocprofv3 counter_collection CSV, per VDA
    kernel, with the derived figures the counters allow: LDS bank-conflict cycles per LDS-active
    cycle, and MFMA TFLOP/s over the dispatch's own duration under the counter pass."""
    rows = _rows(args.summarize_counters)
    acc, dur = {}, {}
    for r in rows:
        name = r["Kernel_Name"]
        if "vda::" not in name:
            continue
        acc.setdefault(name, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            dur.setdefault(name, {})[r.get("Dispatch_Id", len(dur.get(name, {})))] = \
                (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) / 1e3
    print(f"# rocprofv3 counters per dispatch, {args.workload}{' gated' if args.gated else ''}")
    print(f"# command: {args.command}")
    if args.workload.endswith("fp8") and any(c.startswith("MfmaFlops") for k in acc.values() for c in k):
        print("# the statistics kernel's G and Bm run on the FP8 MFMA here, which neither MfmaFlopsBF16 nor "
              "MfmaFlopsF32 counts (its F32 figure is the inverse's updates); MfmaUtil counts every MFMA type")
    counters = sorted({c for k in acc.values() for c in k})
    print(f"{'kernel':<58} " + " ".join(f"{c:>22}" for c in counters) + f" {'us':>9} {'derived':>s}")
    for name, cs in acc.items():
        avg = {c: sum(v) / len(v) for c, v in cs.items()}
        us = sum(dur[name].values()) / len(dur[name]) if name in dur else float("nan")
        derived = []
        if "SQ_LDS_BANK_CONFLICT" in avg and avg.get("SQ_LDS_IDX_ACTIVE"):
            derived.append(f"lds_conflict={100 * avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_LDS_IDX_ACTIVE']:.1f}%")
        for c in avg:
            if c.startswith("MfmaFlops") and us == us and us > 0:
                derived.append(f"{c[9:]}_TFLOP/s={avg[c] / (us * 1e-6) / 1e12:.1f}")
        print(f"{short_name(name)[:58]:<58} " + " ".join(f"{avg.get(c, float('nan')):>22.4g}" for c in counters)
              + f" {us:>9.1f} " + " ".join(derived))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="768p_bf16")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (gradients) after one forward pass")
    ap.add_argument("--gated", action="store_true",
                    help="run the pass with the gated fusion epilogue (seeded synthetic weights)")
    ap.add_argument("--scan-chunk", type=int, default=None,
                    help="frames per chunk of the chunked scan (0: serial; default: the plan's own choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--summarize-stats", metavar="CSV")
    ap.add_argument("--summarize-pmc", nargs=4, metavar="CSV")
    ap.add_argument("--summarize-counters", metavar="CSV",
                    help="counter_collection.csv -> per-kernel averages of every counter")
    ap.add_argument("--command", default="", help="command line recorded in summaries")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the VDA path is benchmarked on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    if args.summarize_stats:
        return summarize_stats(args)
    if args.summarize_pmc:
        return summarize_pmc(args)
    if args.summarize_counters:
        return summarize_counters(args)
    if args.copy_probe:
        return copy_probe(args)
    if args.backward:
        return run_backward(args)
    run(args)


if __name__ == "__main__":
    main()
