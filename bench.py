"""Benchmark of the VC-Attention forward pass on one MI355X.

One step = the whole hot path on one batch of synthetic input already in
HBM: vc_prepare_v (k-means reorder, block means, E4M3 residual),
vc_prepare_qk (per-block E4M3 Q and gathered K) and vc_attention_fwd (the
fused FP8 kernel).  Throughput is attention FLOP per step, 4*B*H*S^2*D,
divided by the step time.

Default workload: B=1, S=73397, H=56, D=128, bf16 (the MiniMax-H3-shaped
layer; "Open VC Attention", Description), V-Smooth k=32, T=5.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0          # MI355X dense FP8 (E4M3) MFMA, published
PEAK_HBM_GBS = 8000.0


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, help="synthetic workload id (3, 4 or 5)")
    ap.add_argument("--heads", type=int, default=None, help="override H (config 4: 7, 14 or 56)")
    ap.add_argument("--seq", type=int, default=None, help="override S")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=6144, help="query rows in the oracle's timed sample")
    ap.add_argument("--cpu-threads", type=int, default=None,
                    help="cap the oracle's BLAS threads (default: all the host gives it)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (for scaling HBM byte counters) and exit")
    ap.add_argument("--hold", type=float, default=0.0, metavar="SECONDS",
                    help="after the timed steps, keep launching the attention kernel for SECONDS "
                         "(a steady load for sampling power and clocks with amd-smi)")
    ap.add_argument("--v-format", choices=["e4m3", "mxfp4"], default="e4m3",
                    help="residual format of V-Smooth: E4M3 with a per-head scale (the default), or the 4-bit "
                         "MXFP4 variant (E2M1 with a power-of-two scale per 32-key group; no repair)")
    ap.add_argument("--ablation-exp", action="store_true",
                    help="also time the attention kernel of libvc_ablation_exp.so (FP32 exponential + E4M3 cast "
                         "instead of ExpCast) on the same prepared workspace")
    ap.add_argument("--library", choices=["main", "ablation-exp"], default="main",
                    help="run every call through libvc.so (the default) or through the measurement build "
                         "libvc_ablation_exp.so (FP32 exponential + E4M3 cast in place of ExpCast), e.g. to "
                         "collect its instruction counters")
    ap.add_argument("--graph", action="store_true",
                    help="also capture the full call once into a HIP graph (the library allocates, clears and "
                         "synchronises nothing, so it captures as is) and time its replays")
    ap.add_argument("--traffic-json", default=os.path.join(ROOT, "profiles", "attn_fwd_traffic.json"),
                    help="HBM bytes per attention launch measured with rocprofv3 counters")
    return ap.parse_args()


def _code_only(text: str) -> str:
    """C++ source without comments and blank lines (the attention sources
    hold no string literal with comment markers)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def attention_kernels(w) -> str:
    """The kernels vc_attention_fwd launches for workload w (the library's attn_split rule)."""
    nblk = -(-w.S // 128)
    if w.repair_budget == 0 and -(-nblk // 16) == 2 and w.B * w.H * nblk <= 256:
        return "vc_attention_fwd (k_vc_attn_halves: one workgroup per query block, keys in two halves)"
    return "vc_attention_fwd (k_vc_attn_fwd + k_vc_attn_tail + k_vc_attn_merge)"


def kernel_sources_sha256() -> str:
    """Hash of the attention kernels' code (comments and blank lines left
    out, so a comment edit keeps a traffic record taken on the same code)."""
    h = hashlib.sha256()
    for f in ("vc_attn.hip", "vc_common.hpp", "vc_kernels.hpp"):
        with open(os.path.join(ROOT, "bit_attention_video_vc_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def traffic_bytes(path: str, key: str):
    """HBM bytes per attention call (the kernels of vc_attention_fwd,
    FETCH_SIZE and WRITE_SIZE scaled by a device copy's readings) from the
    rocprofv3 counter summary, or None if there is none for this workload or
    the kernel sources changed since."""
    try:
        with open(path) as fh:
            rec = json.load(fh).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, q, k, v, rows_n: int, threads_cap: int | None = None) -> dict:
    """The oracle, as is, on one head: full prepare plus a sample of query rows."""
    if threads_cap is not None:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=threads_cap):
            return cpu_baseline(w, q, k, v, rows_n)
    from threadpoolctl import threadpool_info

    from oracle import vc_oracle as O
    import synth

    qn = q[0, :, 0].double().cpu().numpy()
    kn = k[0, :, 0].double().cpu().numpy()
    vn = v[0, :, 0].double().cpu().numpy()
    S = w.S
    rows = synth.sample_rows(S, rows_n).numpy()
    t0 = time.perf_counter()
    hv = O.prepare_v_head(vn, k=w.k, iters=w.iters, repair_budget=w.repair_budget)
    hq = O.prepare_qk_head(qn, kn, hv.perm)
    t1 = time.perf_counter()
    O.attend_head(hq, hv, rows)
    t2 = time.perf_counter()
    t_full_head = (t1 - t0) + (t2 - t1) * S / rows.size       # labelled extrapolation
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    tflops = 4.0 * S * S * w.D / t_full_head / 1e12
    return {
        "value": tflops,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"one head (b=0,h=0) of the same workload: full prepare_v+prepare_qk "
                   f"({t1 - t0:.2f} s) plus attention for {rows.size} sampled query rows ({t2 - t1:.2f} s); "
                   f"value = 4*S^2*D / (t_prepare + t_rows*S/{rows.size}) (extrapolated to the full head)"),
        "host_cpus": os.cpu_count(),
    }


def prepare_report(w, prep_v_ms: float, prep_qk_ms: float) -> dict:
    """Prepare calls (HIP events on the launch stream, average over the timed
    steps) with their algorithmic HBM bytes: per input element, Q and K are
    read once (2 B) and written as E4M3 (1 B); V is read in each of the T+1
    k-means assignment passes, by the block-mean pass and by the quantise
    pass (2 B each) and written once (1 B): 2T+7 bytes."""
    n = w.B * w.H * w.S * w.D
    v_bytes = (2 * w.iters + 7) * n
    qk_bytes = 6 * n
    return {"prepare_v_ms": round(prep_v_ms, 4), "prepare_qk_ms": round(prep_qk_ms, 4),
            "prepare_v_algorithmic_GBps": round(v_bytes / (prep_v_ms * 1e-3) / 1e9, 1),
            "prepare_qk_algorithmic_GBps": round(qk_bytes / (prep_qk_ms * 1e-3) / 1e9, 1),
            "bytes_model": "V (2T+7) B/element, Q and K 3 B/element each"}


def main() -> int:
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(attention heads would shard across GPUs with no exchange; that path is not built)", file=sys.stderr)
        return 2
    import torch

    import bit_attention_video_vc_amd as vc
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.library == "ablation-exp":
        vc.use_library(vc.ablation_exp_lib_path)
        log(f"library: {vc.lib().vc_version().decode()} (measurement build, not the method)")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {n} bytes device to device")
        return 0
    kw = {}
    if args.heads is not None:
        kw["H"] = args.heads
    if args.seq is not None:
        kw["S"] = args.seq
    w = synth.workload(args.config, **kw)
    log(f"workload {w.name}: B={w.B} H={w.H} S={w.S} D={w.D} {w.dtype} k={w.k} T={w.iters} beta={w.repair_budget}")
    t0 = time.time()
    q, k, v = synth.generate(w, "cpu")
    log(f"generated inputs on the host in {time.time() - t0:.1f} s")
    qd, kd, vd = (t.to("cuda") for t in (q, k, v))
    torch.cuda.synchronize()

    v_fmt = vc.VC_V_MXFP4 if args.v_format == "mxfp4" else vc.VC_V_E4M3
    if v_fmt == vc.VC_V_MXFP4 and w.repair_budget > 0:
        print("bench.py: the MXFP4 residual has no repair; pick a workload without it", file=sys.stderr)
        return 2
    opts = vc.v_opts(True, w.k, w.iters, 0, w.repair_budget, v_fmt)
    ws = vc.alloc_workspace(vd, opts)
    out = torch.empty(qd.shape, dtype=torch.bfloat16, device="cuda")
    lay = vc.vc_workspace_layout(vd, opts)
    log(f"workspace {lay.total / 2**30:.2f} GiB")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        # events (on the launch stream): before prepare_v, after it, after
        # prepare_qk, after the attention kernel
        if ev is not None:
            ev[0].record(stream)
        vc.vc_prepare_v(vd, opts, ws, stream)
        if ev is not None:
            ev[1].record(stream)
        vc.vc_prepare_qk(qd, kd, opts, ws, stream)
        if ev is not None:
            ev[2].record(stream)
        vc.vc_attention_fwd(out, opts, ws, 0.0, stream)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup} done")

    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    attn_ms = [e[2].elapsed_time(e[3]) for e in evs]
    prep_v_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / len(evs)
    prep_qk_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / len(evs)
    log(f"timed {args.steps} steps in {t_total:.3f} s")

    ms_per_step = 1e3 * t_total / args.steps
    flops = w.flops
    value = flops / (ms_per_step * 1e-3) / 1e12
    attn_avg_ms = sum(attn_ms) / len(attn_ms)
    attn_tflops = flops / (attn_avg_ms * 1e-3) / 1e12

    traffic = traffic_bytes(args.traffic_json, f"B{w.B}_H{w.H}_S{w.S}")

    res = {
        "metric": "FP8 attention fwd TFLOPS + % of MI355X FP8 MFMA peak at S~73k, D=128",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: B={w.B} S={w.S} H={w.H} D={w.D} {str(w.dtype).replace('torch.', '')} in, bf16 out, "
                        f"non-causal, V-Smooth k={w.k} T={w.iters}, repair={w.repair_budget}"
                        + (", 4-bit MXFP4 residual" if v_fmt == vc.VC_V_MXFP4 else ""),
            "step": "full call: vc_prepare_v + vc_prepare_qk + vc_attention_fwd",
            "flop_per_step": flops,
            "parallelism": "single GPU",
        },
        "pct_of_fp8_peak_full_call": round(100 * value / PEAK_FP8_TFLOPS, 2),
        "kernel_only": {"tflops": round(attn_tflops, 2), "avg_ms": round(attn_avg_ms, 4),
                        "median_ms": round(statistics.median(attn_ms), 4), "min_ms": round(min(attn_ms), 4),
                        "pct_of_fp8_peak": round(100 * attn_tflops / PEAK_FP8_TFLOPS, 2)},
        "prepare_ms_per_step": round(ms_per_step - attn_avg_ms, 3),
        "prepare": prepare_report(w, prep_v_ms, prep_qk_ms),
        "device": {"name": torch.cuda.get_device_name(),
                   "arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", None),
                   "compute_units": torch.cuda.get_device_properties(0).multi_processor_count},
        "roofline": {
            # the attention call: whole work items, the cut last round, the merge;
            # or, for a short launch, the one-workgroup-per-query-block form
            "kernel": attention_kernels(w),
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_FP8_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    if args.graph:
        res["graph"] = graph_replay(w, vd, qd, kd, opts, ws, out, args.steps)
    if args.ablation_exp:
        main_lib = vc.lib_path
        vc.use_library(vc.ablation_exp_lib_path)
        log(f"ablation build: {vc.lib().vc_version().decode()}")
        for _ in range(2):
            vc.vc_attention_fwd(out, opts, ws, 0.0, stream)
        abl = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
        for a, b in abl:
            a.record(stream)
            vc.vc_attention_fwd(out, opts, ws, 0.0, stream)
            b.record(stream)
        torch.cuda.synchronize()
        abl_ms = sum(a.elapsed_time(b) for a, b in abl) / len(abl)
        vc.use_library(main_lib)
        # the ExpCast kernel again, right after, on the same box state
        for a, b in abl:
            a.record(stream)
            vc.vc_attention_fwd(out, opts, ws, 0.0, stream)
            b.record(stream)
        torch.cuda.synchronize()
        ref_ms = sum(a.elapsed_time(b) for a, b in abl) / len(abl)
        res["ablation_exp_cast"] = {
            "what": "attention kernel with an FP32 exponential (v_exp_f32) and an E4M3 cast in place of ExpCast",
            "kernel_ms": round(abl_ms, 4), "tflops": round(flops / (abl_ms * 1e-3) / 1e12, 2),
            "expcast_kernel_ms": round(ref_ms, 4), "expcast_speedup": round(abl_ms / ref_ms, 4)}
    if args.hold > 0:
        n_hold, t_hold0 = 0, time.perf_counter()
        while time.perf_counter() - t_hold0 < args.hold:
            for _ in range(10):
                vc.vc_attention_fwd(out, opts, ws, 0.0, stream)
            torch.cuda.synchronize()
            n_hold += 10
            log(f"hold: {n_hold} launches")
        t_hold = time.perf_counter() - t_hold0
        res["hold"] = {"seconds": round(t_hold, 2), "launches": n_hold, "avg_ms": round(1e3 * t_hold / n_hold, 3)}
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample ...")
        res["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_rows, args.cpu_threads)
    print(json.dumps(res), flush=True)
    return 0


def graph_replay(w, vd, qd, kd, opts, ws, out, steps: int) -> dict:
    """The full call recorded once into a HIP graph (torch.cuda.CUDAGraph) and
    replayed: the launch gaps between the ~15 kernels of a short call go away.
    The replay's output is compared bit for bit with the eager call's."""
    import torch
    import bit_attention_video_vc_amd as vc
    eager = out.clone()

    def full_call(s):
        vc.vc_prepare_v(vd, opts, ws, s)
        vc.vc_prepare_qk(qd, kd, opts, ws, s)
        vc.vc_attention_fwd(out, opts, ws, 0.0, s)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        full_call(side)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        full_call(torch.cuda.current_stream())
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / steps
    log(f"graph replay: {ms:.3f} ms per full call")
    return {"what": "the same full call captured once into a HIP graph and replayed",
            "ms_per_step": round(ms, 4), "tflops": round(w.flops / (ms * 1e-3) / 1e12, 2),
            "identical_to_eager": bool(torch.equal(out, eager))}


if __name__ == "__main__":
    sys.exit(main())
