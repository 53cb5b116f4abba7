"""Tuner for the HCGR op's plan table (run on the GPU).

    python -m skinny_gemm_hcgr_amd.tune --out plans.json [--tokens 1,32,1024]
        [--hc 4 --hs 2560 --r 320] [--merged] [--reps 30]

For each token count (a key), every plan the library can run at that size
(``hcgr_plan_candidates``) is run on seeded random inputs and checked against
the library's own heuristic plan on the same inputs: outputs must be finite,
R2 bit-identical (every plan forms it with the same arithmetic), rrms within
1e-5 relative and inj_next and x within 1e-2 of max|ref| plus 1e-2 relative.
A candidate that fails is rejected and reported. The fastest passing
candidate is then timed against the heuristic plan in six alternating
rounds; it becomes the key's entry unless the heuristic is within 4% of it
(the run-to-run spread measured on MI355X is 2-4%) or it is the heuristic's
own plan (then the entry is marked heuristic).
Timing: median of rounds of ``--reps`` back-to-back calls, rotating over
enough complete sets (inputs, outputs, weights and workspace) that together
exceed the 256 MB Infinity Cache, as the benchmark does: with one set at a
few thousand tokens R2 stays cached between calls, which favours plans that
rely on it (at M = 4096 the staged up kernel read 7% faster than the
heuristic that way and 5% slower on cold sets), and a workspace shared by
the sets keeps the chunk partials cached, which favours plans with more of
them (at M = 4096 a two-segment plan read 4% faster than the heuristic with
one workspace and 1-3% slower with one per set). The table is written
atomically, and not at all if any key is left without a passing candidate.
The table format and the lookup rule (nearest key in log space, the
heuristic below the smallest key) follow the tuned table of the aiter pull
request's "PR Self-Review" section.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

MARGIN = 1.04  # a candidate must beat the heuristic by 4%: run-to-run spread on the box is 2-4%
DEFAULT_TOKENS = [1, 2, 4, 8, 16, 32, 64, 96, 128, 192, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536]
CACHE_BYTES = 256 << 20


def _inputs(torch, cfg, M, seed, nw):
    """Seeded inputs and nw copies of the weights (bf16, N(0,1) activations,
    weights scaled as a trained projection would be). nw is 1 for the tuner,
    which rotates whole sets instead."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    K, hs, hc, r = cfg.k, cfg.hs, cfg.hc, cfg.r

    def n(*shape, std=1.0):
        return (torch.randn(*shape, generator=g) * std).to(torch.bfloat16).cuda()

    inp = {"R": n(M, K), "y": n(M, hs), "inj": n(M, hc)}
    ws = []
    for _ in range(nw):
        wn = n(cfg.wnorm_len or hs, std=0.1)
        wd, wi = n(r, K, std=K ** -0.5), n(hc, K, std=K ** -0.5)
        w = {"wnorm": wn, "wu": n(K, r, std=r ** -0.5)}
        if cfg.merged:
            wm = torch.zeros(cfg.n_pad, K, dtype=torch.float32, device="cuda")
            wm[:r], wm[r:r + hc] = wd.float(), wi.float()
            f = wn.float() if wn.numel() == K else wn.float().repeat(K // wn.numel())
            w["wd"], w["wi"] = (wm * (1.0 + f)).to(torch.bfloat16), None
        else:
            w["wd"], w["wi"] = wd, wi
        ws.append(w)
    return inp, ws


def _agree(torch, out, ref):
    """None when out matches ref within the tuner's bounds, else the reason."""
    for k in ("R2", "rrms", "inj_next", "x"):
        if not torch.isfinite(out[k].float()).all():
            return f"non-finite {k}"
    if not torch.equal(out["R2"], ref["R2"]):
        return "R2 differs"
    rel = ((out["rrms"] - ref["rrms"]).abs() / ref["rrms"].abs()).max().item()
    if rel > 1e-5:
        return f"rrms off by {rel:.2e}"
    for k in ("inj_next", "x"):
        a, b = out[k].float(), ref[k].float()
        lim = 1e-2 * b.abs().max() + 1e-2 * b.abs()
        if ((a - b).abs() > lim).any():
            return f"{k} beyond tolerance"
    return None


def tune(cfg, tokens, reps=30, seed=0, log=print):
    import torch
    import skinny_gemm_hcgr_amd as H
    op = H.HCGR(cfg, 0)
    stream = torch.cuda.current_stream().cuda_stream
    entries, failures = [], []
    wbytes = (cfg.r + cfg.hc) * cfg.k * 2 + cfg.k * cfg.r * 2
    per_token = cfg.k * 4 + cfg.hs * 4 + cfg.hc * 8  # R, R2, y, x, inj, inj_next, rrms
    for M in tokens:
        nset = max(1, min(32, math.ceil(1.25 * CACHE_BYTES / (wbytes + M * per_token))))
        sets = []
        for j in range(nset):
            inp, w = _inputs(torch, cfg, M, seed + M + 7919 * j, 1)
            sets.append((inp, w[0], op.alloc_outputs(M)))
        cands = H.hcgr_plan_candidates(cfg, M)
        choices = [{"tokens": M, "kind": H.HCGR_PLAN_HEURISTIC}] + cands
        need = max(H.hcgr_workspace_size_table(cfg, [c], M) for c in choices)
        wss = [H.new_workspace(need) for _ in range(nset)]  # one per set, as the benchmark's
        outs = sets[0][2]  # the set every plan's result is checked on

        def run(i):
            inp, w, o = sets[i % nset]
            ws = wss[i % nset]
            H.hcgr_forward(op.handle, inp["R"], inp["y"], inp["inj"], inp["inj"].stride(0), w["wnorm"], w["wd"],
                           w["wi"], w["wu"], M, o["R2"], o["rrms"], o["inj_next"], o["ld_inj_next"],
                           o["x"], ws, ws.numel(), stream)

        op.set_plan_table([])
        for i in range(20):  # warm-up: the first plan timed must not pay for first launches
            run(i)
        torch.cuda.synchronize()
        def time_round():
            for i in range(3):
                run(i)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(reps):
                run(i)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) * 1e3 / reps

        ref = None
        results = []
        for c in choices:
            op.set_plan_table([c] if c["kind"] != H.HCGR_PLAN_HEURISTIC else [])
            run(0)
            torch.cuda.synchronize()
            got = {k: outs[k].clone() for k in ("R2", "rrms", "inj_next", "x")}
            if ref is None:
                ref = got
            else:
                why = _agree(torch, got, ref)
                if why:
                    failures.append((M, c, why))
                    log(f"[tune] M={M} reject {c}: {why}")
                    continue
            results.append((sorted(time_round() for _ in range(3))[1], c))
        # final decision on paired measurements: the heuristic and the best
        # candidate timed alternately (a plan timed early in a sweep can read
        # slower while the clocks settle), and a candidate whose plan is the
        # heuristic's own counts as the heuristic
        best = min(results, key=lambda t: t[0])[1]
        heur_desc = H.hcgr_describe_plan(cfg, M)
        th, tb = [], []
        for _ in range(6):
            op.set_plan_table([])
            th.append(time_round())
            op.set_plan_table([best] if best["kind"] != H.HCGR_PLAN_HEURISTIC else [])
            tb.append(time_round())
        op.set_plan_table([])
        heur_us, best_us = sorted(th)[2], sorted(tb)[2]
        if (best["kind"] == H.HCGR_PLAN_HEURISTIC or best_us >= heur_us / MARGIN
                or H.hcgr_plan_lookup(cfg, [best], M)[1] == heur_desc):
            best, best_us = results[0][1], heur_us
        entry = {k: int(best.get(k, 0)) for k in H.PLAN_FIELDS}
        entry.update({"us": round(best_us, 3), "heuristic_us": round(heur_us, 3), "candidates": len(results)})
        entries.append(entry)
        log(f"[tune] M={M}: heuristic {heur_us:.2f} us, chosen {best_us:.2f} us "
            f"({'heuristic' if entry['kind'] == H.HCGR_PLAN_HEURISTIC else H.hcgr_plan_lookup(cfg, [entry], M)[1]})")
        del wss, outs, sets
        torch.cuda.empty_cache()
    op.close()
    return entries, failures


def write_table(path, cfg, entries):
    import torch
    doc = {"config": {"hc": cfg.hc, "hs": cfg.hs, "r": cfg.r, "wnorm_len": cfg.wnorm_len or cfg.hs,
                      "weight_layout": cfg.weight_layout, "n_pad": cfg.n_pad},
           "device": torch.cuda.get_device_properties(0).gcnArchName.split(":")[0],
           "lookup": "nearest key in log space; the heuristic below the smallest key and for heuristic entries",
           "entries": entries}
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        json.dump(doc, f, indent=1)
    os.replace(tmp, path)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--out", required=True)
    ap.add_argument("--tokens", default=",".join(map(str, DEFAULT_TOKENS)))
    ap.add_argument("--hc", type=int, default=4)
    ap.add_argument("--hs", type=int, default=2560)
    ap.add_argument("--r", type=int, default=320)
    ap.add_argument("--merged", action="store_true", help="merged/folded down-inject weight (n_pad = r + hc rounded to 16)")
    ap.add_argument("--reps", type=int, default=30)
    args = ap.parse_args(argv)
    import skinny_gemm_hcgr_amd as H
    n_pad = (args.r + args.hc + 15) // 16 * 16
    cfg = H.Config(hc=args.hc, hs=args.hs, r=args.r,
                   weight_layout=H.HCGR_WEIGHTS_MERGED_FOLDED if args.merged else H.HCGR_WEIGHTS_SEPARATE,
                   n_pad=n_pad if args.merged else 0)
    tokens = sorted({int(t) for t in args.tokens.split(",") if t})
    t0 = time.time()
    entries, failures = tune(cfg, tokens, reps=args.reps)
    if len(entries) != len(tokens):
        print("[tune] some token counts have no passing plan; no table written", file=sys.stderr)
        return 1
    write_table(args.out, cfg, entries)
    print(f"[tune] wrote {args.out}: {len(entries)} entries, {len(failures)} rejected candidates, "
          f"{time.time() - t0:.0f} s", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
