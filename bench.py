#!/usr/bin/env python3
"""Benchmark of the Hyper-Connection Gated Residual op on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-sweep] [--no-cpu] [--warm]
    python bench.py --entry combine|mix [--entry-m M] [--steps K]

A step is one hcgr_forward call (all three kernels) over one batch of M
tokens. The headline line is the decode batch M=32 (HC=4, HS=2560, r=320,
bf16, separate Wd/Wi). Timing:
  * the K timed steps are queued behind a GPU spin kernel, so the host has
    enqueued all of them before the GPU starts; HIP events bracket the K
    steps on the stream the library launches on (device back-to-back time,
    like a graph replay; host launch overhead is reported separately);
  * "cold": every step reads its own copy of the weights and activations,
    rotating over enough sets to exceed the 256 MB Infinity Cache, so the
    weights come from HBM as they would when other layers run in between;
    "warm" re-reads one set.
  * per-kernel durations come from the start/end HIP events that
    hcgr_forward_timed takes around each kernel on the same stream.
Plans: the tuned tables shipped with the package (skinny_gemm_hcgr_amd/plans,
written by skinny_gemm_hcgr_amd.tune on an MI355X); --heuristic plans by the
library's own heuristic instead.
Inputs are seeded synthetic data (synth/) with the study's distributions.
Prints ONE JSON line on stdout; --json-out also writes it (and the sweep) to a file.
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

METRIC = "µs/call & tokens/s of HC gated-residual op, M=1..65536; % HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
CACHE_BYTES = 256 << 20      # Infinity Cache; rotating sets exceed it
HC, HS, R_LOW = 4, 2560, 320
K = HC * HS


def op_bytes(M, merged=False, hc=HC, hs=HS, r=R_LOW):
    """Algorithmic bytes of one call: weights once (Wd, Wi or the r + HC used rows
    of Wm, Wu, Wnorm) + per token R, y, inj in and R2, rrms, inj_next, x out."""
    k = hc * hs
    w = (r + hc) * k * 2 + k * r * 2 + (0 if merged else hs * 2)
    if merged:
        w += hs * 2  # the up kernel still reads Wnorm
    return w + M * (k * 2 + hs * 2 + hc * 2 + k * 2 + hc * 4 + hc * 2 + hs * 2)


def op_flops(M, hc=HC, hs=HS, r=R_LOW):
    k = hc * hs
    return M * 2 * (r + hc) * k + M * 2 * r * k


def kernel_bytes(name, M, merged=False, plan=""):
    """Algorithmic bytes per launch of each kernel: what it must read and write
    at least, given what it receives and hands on (weights once per launch)."""
    wdown = (R_LOW + HC) * K * 2 + (0 if merged else HS * 2)
    act_in = K * 2 + HS * 2 + HC * 2          # R, y, inj
    if name == "hcgr_k1_dec":
        return wdown + M * (act_in + K * 2)     # + R2 out
    if name == "hcgr_k1_fuse":                  # + R2, rrms, inj_next out (the reduction is in-kernel)
        return wdown + M * (act_in + K * 2 + HC * 4 + HC * 2)
    if name == "hcgr_dec_persist":              # the whole op in one kernel
        return op_bytes(M, merged)
    if name == "hcgr_k1_reduce":
        return M * (HC * 4 + HC * 2)            # rrms, inj_next out
    if name in ("hcgr_k1_full", "hcgr_k1_tile"):
        writes_inj = "plan=full" in plan or "streams/wg=4" in plan
        out = K * 2 + HC * 4 + (HC * 2 if writes_inj else 0)
        return wdown + M * (act_in + out)
    if name == "hcgr_k1_sum":
        return M * HC * 2                       # inj_next out
    if name in ("hcgr_k2_dec", "hcgr_k2_decg", "hcgr_k2_stage", "hcgr_k2_sweep", "hcgr_k2_sweep2"):
        return K * R_LOW * 2 + HS * 2 + M * (K * 2 + HC * 4 + HS * 2)  # Wu, Wnorm; R2, rrms in; x out
    raise KeyError(name)


def kernel_flops(name, M):
    if name in ("hcgr_k1_dec", "hcgr_k1_fuse", "hcgr_k1_full", "hcgr_k1_tile"):
        return M * 2 * (R_LOW + HC) * K
    if name == "hcgr_dec_persist":
        return op_flops(M)
    if name in ("hcgr_k2_dec", "hcgr_k2_decg", "hcgr_k2_stage", "hcgr_k2_sweep", "hcgr_k2_sweep2"):
        return M * 2 * R_LOW * K
    return 0


def stage_names(plan: str):
    """Kernels between the four timing marks of hcgr_forward_timed (None where
    a plan has no kernel between two marks)."""
    if "plan=fused" in plan:
        return ("hcgr_k1_fuse", None, "hcgr_k2_decg")
    if "plan=persistent" in plan:
        return ("hcgr_dec_persist", None, None)
    if "plan=split" in plan:
        return ("hcgr_k1_dec", "hcgr_k1_reduce", "hcgr_k2_dec")
    up = ("hcgr_k2_sweep2" if "k2_sweep2" in plan else "hcgr_k2_sweep" if "k2_sweep" in plan else
          "hcgr_k2_gen" if "k2_gen" in plan else "hcgr_k2_stage")
    if "plan=tile" in plan:
        return ("hcgr_k1_tile", "hcgr_k1_sum" if "streams/wg=1" in plan else None, up)
    if "plan=stream" in plan:
        return ("hcgr_k1_full", "hcgr_k1_sum", up)
    return ("hcgr_k1_full", None, up)


class Sets:
    """NB independent buffer sets (inputs, weights, outputs, workspace) for M tokens."""

    def __init__(self, H, op, M, nb, merged=False, scale_stream0=1.0, seed0=0, entry="forward", hc=HC):
        import torch
        import synth
        self.M, self.nb, self.merged, self.entry = M, nb, merged, entry
        sh = synth.Shape(hc, HS, R_LOW)
        self.sets = []
        for i in range(nb):
            inp = synth.make_inputs(M, sh, seed=seed0 + i, device="cuda", scale_stream0=scale_stream0)
            if merged:
                inp["wd"] = synth.fold_merged_weight(inp["wd"], inp["wi"], inp["wnorm"], 336, HS)
                inp["wi"] = None
            out = op.alloc_outputs(M)
            ws = H.new_workspace(H.hcgr_workspace_size(op.handle, M))
            self.sets.append((inp, out, ws))

    def call(self, H, op, i, stream, events=None):
        inp, out, ws = self.sets[i % self.nb]
        if self.entry == "combine":
            H.hcgr_combine(op.handle, inp["R"], inp["y"], inp["inj"], inp["inj"].stride(0), self.M, out["R2"], stream)
            return
        if self.entry == "mix":
            H.hcgr_mix(op.handle, inp["R"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], self.M, out["rrms"],
                       out["inj_next"], out["ld_inj_next"], out["x"], ws, ws.numel(), stream)
            return
        args = (op.handle, inp["R"], inp["y"], inp["inj"], inp["inj"].stride(0), inp["wnorm"], inp["wd"], inp["wi"],
                inp["wu"], self.M, out["R2"], out["rrms"], out["inj_next"], out["ld_inj_next"], out["x"], ws,
                ws.numel(), stream)
        if events is None:
            H.hcgr_forward(*args)
        else:
            H.hcgr_forward_timed(*args, events)


def set_count(M, merged=False, cold=True, hc=HC):
    if not cold:
        return 1
    per = op_bytes(M, merged, hc) + M * (hc * HS * 2 + HS * 2)  # + outputs written
    return max(1, min(64, math.ceil(1.25 * CACHE_BYTES / per)))


def _spin(torch, us):
    # torch's bounded spin kernel (clock cycles at ~2.4 GHz); holds the queue
    torch.cuda._sleep(int(us * 2400))


def time_calls(H, op, sets, steps, warmup, stream):
    """Device time per call (µs) for `steps` back-to-back calls, plus the host
    enqueue time per call."""
    import torch
    for i in range(warmup):
        sets.call(H, op, i, stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(min(steps, 20)):
        sets.call(H, op, i, stream)
    host_us = (time.perf_counter() - t0) / min(steps, 20) * 1e6
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    _spin(torch, host_us * steps * 1.5 + 2000)
    start.record()
    for i in range(steps):
        sets.call(H, op, i, stream)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / steps, host_us


def time_call_stats(H, op, sets, stream, n=60, sweeps=3):
    """The statistic of the pages' benchmark table: each call of a sweep timed
    on its own (HIP events between back-to-back calls, all queued behind a GPU
    spin before the first runs), the median of n calls per sweep, then the
    median of the sweeps and their spread (max - min) / median."""
    import torch
    meds = []
    for _ in range(sweeps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        torch.cuda.synchronize()
        _spin(torch, 40 * n + 2000)
        ev[0].record()
        for i in range(n):
            sets.call(H, op, i, stream)
            ev[i + 1].record()
        torch.cuda.synchronize()
        d = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n))
        meds.append(d[n // 2] if n % 2 else 0.5 * (d[n // 2 - 1] + d[n // 2]))
    med = sorted(meds)[len(meds) // 2]
    return {"median_us": round(med, 3), "sweep_medians_us": [round(m, 3) for m in meds],
            "spread": round((max(meds) - min(meds)) / med, 4), "calls_per_sweep": n, "sweeps": sweeps}


def time_kernels(H, op, sets, steps, stream, host_us):
    """Average duration (µs) of each of the three kernels over `steps` calls,
    from the start/end HIP events hcgr_forward_timed takes around each kernel
    on the launch stream (kernel execution only, no dispatch gaps)."""
    import torch
    evs = []
    for _ in range(steps):
        row = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        for e in row:
            e.record()  # materialise the hipEvent_t
        evs.append(row)
    torch.cuda.synchronize()
    _spin(torch, (host_us + 20) * steps * 1.5 + 2000)
    for i in range(steps):
        sets.call(H, op, i, stream, [e.cuda_event for e in evs[i]])
    torch.cuda.synchronize()
    sums = [0.0, 0.0, 0.0]
    for row in evs:
        for j in range(3):  # start and end of stage j's kernel
            sums[j] += row[2 * j].elapsed_time(row[2 * j + 1]) * 1e3
    names = stage_names(op.describe(sets.M))
    return {names[j]: sums[j] / steps for j in range(3) if names[j]}


def time_graph(H, op, sets, replays, stream):
    """µs per call when `sets.nb` calls are captured into one HIP graph and replayed."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(sets.nb):
            sets.call(H, op, i, s.cuda_stream)
        with torch.cuda.graph(g, stream=s):
            for i in range(sets.nb):
                sets.call(H, op, i, s.cuda_stream)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    _spin(torch, 40 * replays + 2000)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    us = start.elapsed_time(end) * 1e3 / (replays * sets.nb)
    del g
    return us


def measure_copy_gbs(torch, nbytes=1 << 30, reps=10):
    """Achievable HBM bandwidth on this machine: read + write bytes per second of a
    plain device-to-device copy of nbytes (median of reps)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / sorted(times)[len(times) // 2] / 1e9


def measure_gemm_tflops(torch, n=8192, reps=10):
    """bf16 dense GEMM rate of the platform's library GEMM (torch.matmul on an
    n x n x n product): the achievable matrix-core rate on this machine, beside
    the published 2.5 PFLOP/s. Median of reps event-timed calls."""
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.matmul(a, b)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    del a, b
    torch.cuda.empty_cache()
    return 2.0 * n ** 3 / sorted(times)[len(times) // 2] / 1e12


def kernel_source_digest():
    """Digest of the kernel sources; a counter summary taken on other sources no longer applies."""
    import glob
    import hashlib
    h = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "skinny_gemm_hcgr_amd", "csrc", "*"))):
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from a committed rocprofv3
    counter summary (profiles/*_traffic.md: FETCH_SIZE and WRITE_SIZE scaled
    by a copy kernel of known size), or None when there is none or the kernel
    sources have changed since the counters were taken."""
    import glob
    import re
    digest = kernel_source_digest()
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.md"))):
        with open(f) as fh:
            text = fh.read()
        for block in re.findall(r"```json\n(.*?)\n```", text, re.S):
            try:
                d = json.loads(block)
            except ValueError:
                continue
            if d.get("workload") == workload and d.get("kernel") == kernel and d.get("source_digest") == digest:
                return d.get("traffic_bytes_per_launch")
    return None


def roofline_entry(name, M, us, merged, plan, workload):
    b = kernel_bytes(name, M, merged, plan)
    gbs = b / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name, workload), "kernel": name,
            "avg_us": round(us, 3), "alg_bytes_per_launch": b, "flops_per_launch": kernel_flops(name, M),
            "source_digest": kernel_source_digest()}


def run_workload(H, op_sep, op_merged, name, M, merged, scale0, steps, warmup, cold, stream, extras=True):
    """Times one workload: K back-to-back calls (the headline), per-kernel
    durations, and with `extras` the pages' per-call statistic and a graph
    replay."""
    op = op_merged if merged else op_sep
    nb = set_count(M, merged, cold)
    sets = Sets(H, op, M, nb, merged=merged, scale_stream0=scale0)
    us, host_us = time_calls(H, op, sets, steps, warmup, stream)
    kern = time_kernels(H, op, sets, max(8, min(steps, 200)), stream, host_us)
    stats = time_call_stats(H, op, sets, stream) if extras else None
    graph_us = time_graph(H, op, sets, max(1, min(200, (steps + nb - 1) // nb)), stream) if extras else None
    B, F = op_bytes(M, merged), op_flops(M)
    res = {"workload": name, "M": M, "merged": merged, "buffer_sets": nb,
           "cache": "cold (rotating sets > Infinity Cache)" if nb > 1 else ("warm" if not cold else "single set"),
           "us_per_call": round(us, 3), "us_per_call_graph": round(graph_us, 3) if graph_us else None,
           "per_call_stats": stats,
           "host_enqueue_us_per_call": round(host_us, 2), "tokens_per_s": round(M / (us * 1e-6), 1),
           "op_alg_bytes": B, "op_flops": F,
           "op_hbm_frac": round(B / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
           "op_mfma_frac": round(F / (us * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
           "op_roofline_us": round(max(B / (HBM_PEAK_GBS * 1e9), F / (MFMA_BF16_PEAK_TFLOPS * 1e12)) * 1e6, 3),
           "kernels_us": {k: round(v, 3) for k, v in kern.items()},
           "plan": op.describe(M)}
    res["op_roofline_frac"] = round(res["op_roofline_us"] / us, 4)
    del sets
    return res


def cpu_model():
    """CPU model name and the host's logical core count."""
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    name = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return name, os.cpu_count()


# The oracle's CPU baseline: per workload, the tokens timed with all cores and
# with one thread and the repetitions (median taken). Every step is per token,
# so a row sample of a large workload runs at that workload's per-token cost;
# the samples keep the whole leg to about ten seconds of CPU time.
CPU_PLAN = {1: (1, 5, 1, 5), 32: (32, 5, 32, 3), 1024: (256, 3, 16, 3), 8192: (256, 3, 16, 3),
            65536: (256, 3, 16, 3)}


def cpu_baseline(M_head):
    """The fp64 oracle (as it stands, OpenMP over tokens) on this host's cores:
    µs/call and tokens/s per workload size, all cores and one thread, on the
    same seeded inputs as the GPU run (row samples of the larger sizes)."""
    import oracle
    import synth
    cfg = oracle.OracleConfig()
    wts = synth.make_weights(synth.Shape(HC, HS, R_LOW), seed=0, device="cpu")
    model, ncpu = cpu_model()
    nthreads = oracle.max_threads()
    per_m = []
    head = None
    for M, (n_all, reps_all, n_one, reps_one) in CPU_PLAN.items():
        d = synth.make_inputs(max(n_all, n_one), synth.Shape(HC, HS, R_LOW), seed=0, device="cpu", weights=wts,
                              scale_stream0=8.0 if M == 8192 else 1.0)
        rec = {"M": M}
        for label, n, reps, threads in (("all_cores", n_all, reps_all, 0), ("one_thread", n_one, reps_one, 1)):
            times = []
            for _ in range(reps):
                t0 = time.perf_counter()
                oracle.forward(cfg, d["R"][:n], d["y"][:n], d["inj"][:n], d["wnorm"], d["wd"], d["wi"], d["wu"],
                               threads=threads)
                times.append(time.perf_counter() - t0)
            t = sorted(times)[len(times) // 2]
            rec[label] = {"tokens_timed": n, "reps": reps, "tokens_per_s": round(n / t, 2),
                          "us_per_token": round(t / n * 1e6, 2),
                          "us_per_call_est": round(t / n * M * 1e6, 1), "threads": nthreads if threads == 0 else 1}
        per_m.append(rec)
        if M == M_head:
            head = rec
    if head is None:
        head = per_m[1]
    a = head["all_cores"]
    return {"value": a["tokens_per_s"], "unit": "tokens/s", "cores": a["threads"], "kind": "oracle",
            "sample": f"{a['reps']} runs (median) of {a['tokens_timed']} tokens of the M={head['M']} workload, fp64 "
                      "oracle, OpenMP over tokens on all cores",
            "cpu_model": model, "nproc": ncpu, "per_m": per_m,
            "note": "large M timed on row samples (every step is per token); us_per_call_est = per-token time x M"}


def entry_bytes(entry, M):
    """Algorithmic bytes of one call of the combine-only or mix entry point."""
    if entry == "combine":  # R, y, inj in; R2 out
        return M * (K * 2 + HS * 2 + HC * 2 + K * 2)
    # mix: weights once; R in; rrms, inj_next, x out
    return op_bytes(0) + M * (K * 2 + HC * 4 + HC * 2 + HS * 2)


def run_entry(H, op, entry, M, steps, stream):
    nb = 1 if entry == "combine" else set_count(M)
    sets = Sets(H, op, M, nb, entry=entry)
    us, _ = time_calls(H, op, sets, steps, 5, stream)
    B = entry_bytes(entry, M)
    gbs = B / (us * 1e-6) / 1e9
    del sets
    return {"entry": entry, "M": M, "buffer_sets": nb, "us_per_call": round(us, 3),
            "tokens_per_s": round(M / (us * 1e-6), 1), "alg_bytes": B, "achieved_gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


ENTRY_RUNS = [("combine", 8192), ("combine", 65536), ("mix", 32), ("mix", 8192)]


def run_streams(H, hc, M, steps, stream):
    """The whole op at another stream count (HS = 2560, r = 320) with the plan
    table shipped for that shape (the heuristic where there is none)."""
    op = H.HCGR(H.Config(hc=hc), 0, plan_table="shipped")
    nb = set_count(M, hc=hc)
    sets = Sets(H, op, M, nb, hc=hc)
    us, _ = time_calls(H, op, sets, steps, 5, stream)
    B, F = op_bytes(M, hc=hc), op_flops(M, hc=hc)
    res = {"hc": hc, "M": M, "buffer_sets": nb, "us_per_call": round(us, 3),
           "tokens_per_s": round(M / (us * 1e-6), 1), "op_hbm_frac": round(B / (us * 1e-6) / (HBM_PEAK_GBS * 1e9), 4),
           "op_mfma_frac": round(F / (us * 1e-6) / (MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
           "plan": H.hcgr_describe_plan(op.cfg, M)}
    del sets
    op.close()
    return res


STREAM_RUNS = [(2, 32), (2, 8192), (8, 32), (8, 8192)]

WORKLOADS = {
    "decode_m1": (1, False, 1.0),
    "decode_m32": (32, False, 1.0),
    "merged_m1024": (1024, True, 1.0),
    "prefill_m8192_s0x8": (8192, False, 8.0),
    "prefill_m65536": (65536, False, 1.0),
}
SWEEP_M = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_m32", choices=sorted(WORKLOADS))
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--warm", action="store_true", help="headline on one re-read buffer set")
    ap.add_argument("--cold-only", action="store_true",
                    help="only the headline's cold rotating-set calls (no warm set, graph replay, per-call "
                         "statistic, sweep or CPU leg): the command the kernel traces are taken with")
    ap.add_argument("--heuristic", action="store_true",
                    help="plan by the library's heuristic instead of the tuned tables shipped with the package")
    ap.add_argument("--json-out", default=None)
    ap.add_argument("--entry", choices=("combine", "mix"), default=None,
                    help="only time this entry point at --entry-m tokens (for profiling) and exit")
    ap.add_argument("--entry-m", type=int, default=8192)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run 5 device-to-device copies of BYTES (HBM counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the op is token-parallel and this build has no multi-GPU "
              "path (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import torch
    import skinny_gemm_hcgr_amd as H
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        src = torch.ones(args.copy_probe, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": args.copy_probe, "launches": 5}))
        return
    H.load_library()
    table = None if args.heuristic else "shipped"
    op = H.HCGR(H.Config(), 0, plan_table=table)
    if args.entry:
        r = run_entry(H, op, args.entry, args.entry_m, args.steps, torch.cuda.current_stream().cuda_stream)
        print(json.dumps(r), flush=True)
        return
    opm = H.HCGR(H.Config(weight_layout=H.HCGR_WEIGHTS_MERGED_FOLDED, n_pad=336), 0, plan_table=table)
    plans = "heuristic" if args.heuristic else (os.path.relpath(H.shipped_plan_table(op.cfg), ROOT)
                                                if H.shipped_plan_table(op.cfg) else "heuristic")
    stream = torch.cuda.current_stream().cuda_stream

    M, merged, scale0 = WORKLOADS[args.workload]
    torch.cuda.synchronize()
    if args.cold_only:
        args.no_sweep = args.no_cpu = True
    head = run_workload(H, op, opm, args.workload, M, merged, scale0, args.steps, args.warmup, not args.warm, stream,
                        extras=not args.cold_only)
    warm = None
    if not args.warm and not args.cold_only:
        warm = run_workload(H, op, opm, args.workload, M, merged, scale0, args.steps, args.warmup, False, stream,
                            extras=False)
    torch.cuda.synchronize()
    print(f"[bench] {args.workload}: {head['us_per_call']} us/call ({head['cache']}), kernels {head['kernels_us']}",
          file=sys.stderr, flush=True)

    sweep = []
    if not args.no_sweep:
        named = [(n, *v) for n, v in WORKLOADS.items() if n != args.workload]
        extra = [(f"sweep_m{m}", m, False, 1.0) for m in SWEEP_M if m not in (1, 32, 65536)]
        for name, m, mg, sc in named + extra:
            steps = max(10, min(args.steps, int(2e5 / max(1, m)) + 10))
            r = run_workload(H, op, opm, name, m, mg, sc, steps, 5, True, stream)
            print(f"[bench] {name}: {r['us_per_call']} us/call graph {r['us_per_call_graph']} "
                  f"roofline {r['op_roofline_frac']}", file=sys.stderr, flush=True)
            sweep.append(r)
            torch.cuda.empty_cache()

    entries = []
    if not args.no_sweep:
        for entry, m in ENTRY_RUNS:
            r = run_entry(H, op, entry, m, max(10, min(args.steps, int(2e5 / m) + 10)), stream)
            print(f"[bench] {entry} M={m}: {r['us_per_call']} us/call, {r['achieved_gbs']} GB/s", file=sys.stderr,
                  flush=True)
            entries.append(r)
            torch.cuda.empty_cache()

    streams = []
    if not args.no_sweep:
        for hc, m in STREAM_RUNS:
            r = run_streams(H, hc, m, max(10, min(args.steps, int(2e5 / m) + 10)), stream)
            print(f"[bench] HC={hc} M={m}: {r['us_per_call']} us/call", file=sys.stderr, flush=True)
            streams.append(r)
            torch.cuda.empty_cache()

    dom = max(head["kernels_us"], key=lambda k: head["kernels_us"][k])
    roof = roofline_entry(dom, M, head["kernels_us"][dom], merged, head["plan"], args.workload)
    copy_gbs = measure_copy_gbs(torch)
    gemm_tflops = measure_gemm_tflops(torch)
    roof["frac_of_measured_copy"] = round(roof["achieved"] / copy_gbs, 4)
    line = {"metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(head["us_per_call"] / 1e3, 6),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded SplitMix64/Box-Muller, the study's distributions)",
            "config": {"workload": args.workload, "M": M, "hc": HC, "hs": HS, "r": R_LOW, "eps": 1e-6,
                       "weights": "merged_folded_n336" if merged else "separate",
                       "buffers": head["cache"], "buffer_sets": head["buffer_sets"], "plans": plans},
            "us_per_call": head["us_per_call"], "us_per_call_graph": head["us_per_call_graph"],
            "per_call_stats": head["per_call_stats"],
            "us_per_call_warm": warm["us_per_call"] if warm else None,
            "op_roofline_frac": head["op_roofline_frac"], "op_hbm_frac": head["op_hbm_frac"],
            "kernels_us": head["kernels_us"], "roofline": roof,
            "measured_peaks": {"hbm_copy_gbs": round(copy_gbs, 1), "bf16_gemm_tflops": round(gemm_tflops, 1),
                               "note": "read + write bytes per second of a 1 GiB device copy, and the bf16 rate "
                                       "of an 8192^3 library GEMM (torch.matmul), on this box; op_hbm_frac, "
                                       "op_mfma_frac and roofline.frac use the published 8 TB/s and 2.5 PFLOP/s"},
            "context": {"pages_two_stage_graph_us": {"1": 21.0, "32": 28.8, "1024": 76.3, "8192": 339.2,
                                                     "65536": 2636.4},
                        "note": "page numbers: MI355X, merged/folded weights, graph replay; context only"}}
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(M)
    else:
        line["cpu_baseline"] = None
    if sweep:
        line["sweep"] = [{k: r[k] for k in ("workload", "M", "us_per_call", "us_per_call_graph", "per_call_stats",
                                            "tokens_per_s", "op_roofline_frac", "op_hbm_frac", "op_mfma_frac",
                                            "kernels_us")}
                         for r in sweep]
    if entries:
        line["entries"] = entries
    if streams:
        line["stream_counts"] = [{k: v for k, v in r.items() if k != "plan"} for r in streams]
    if args.json_out:
        with open(args.json_out, "w") as f:
            json.dump({"line": line, "headline": head, "warm": warm, "sweep": sweep}, f, indent=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
