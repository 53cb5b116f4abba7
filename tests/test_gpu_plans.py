"""GPU parity of every plan a tuned table may choose, and of the tuner end to
end: each candidate plan (hcgr_plan_candidates) installed as a one-entry
table must match the fp64 oracle; a table written by
skinny_gemm_hcgr_amd.tune must load and give oracle-matching results at and
between its keys."""
from __future__ import annotations

import os
import tempfile

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_all

pytestmark = pytest.mark.gpu

SHAPE = synth.Shape()


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import skinny_gemm_hcgr_amd as H
    H.load_library()
    return H


@pytest.fixture(scope="module")
def weights():
    return synth.make_weights(SHAPE, seed=0, device="cuda")


def _say(msg):
    print(msg, flush=True)


def sample_rows(M, n=24, seed=3):
    rng = np.random.default_rng(seed)
    rows = {0, M // 2, M - 1} | set(rng.choice(M, size=min(n, M), replace=False).tolist())
    return np.array(sorted(rows))


def run_oracle(inp, rows=None):
    R, y, inj = inp["R"], inp["y"], inp["inj"]
    if rows is not None:
        idx = torch.as_tensor(rows, device="cuda")
        R, y, inj = R[idx], y[idx], inj[idx]
    return oracle.forward(oracle.OracleConfig(), R.cpu(), y.cpu(), inj.cpu(), inp["wnorm"].cpu(), inp["wd"].cpu(),
                          inp["wi"].cpu(), inp["wu"].cpu())


def check_rows(out, ref, rows):
    if rows is None:
        check_all(out, ref)
    else:
        idx = torch.as_tensor(rows, device="cuda")
        check_all({k: out[k][idx] for k in ("R2", "rrms", "inj_next", "x")}, ref)


@pytest.mark.parametrize("M", [1, 32, 100, 300, 4100])
def test_every_candidate_plan(H, weights, M):
    op = H.HCGR(H.Config(), 0)
    inp = synth.make_inputs(M, SHAPE, seed=60 + M, device="cuda", weights=weights)
    rows = None if M <= 300 else sample_rows(M)
    ref = run_oracle(inp, rows)
    cands = H.hcgr_plan_candidates(op.cfg, M)
    _say(f"[plans] M={M}: {len(cands)} candidates")
    for c in cands:
        op.set_plan_table([c])
        desc = op.describe(M)
        _say(f"[plans]   {desc}")
        out = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
        torch.cuda.synchronize()
        try:
            check_rows(out, ref, rows)
        except AssertionError as e:
            raise AssertionError(f"{c} ({desc}): {e}") from None
    op.close()


def test_tuner_end_to_end(H, weights):
    from skinny_gemm_hcgr_amd import tune
    cfg = H.Config()
    entries, failures = tune.tune(cfg, [16, 600], reps=3, log=_say)
    assert len(entries) == 2 and not failures, failures
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "plans.json")
        tune.write_table(path, cfg, entries)
        op = H.HCGR(cfg, 0, plan_table=path)
        with pytest.raises(ValueError):
            H.load_plan_table(path, H.Config(hs=1024))  # tuned for another shape
    for M in (16, 100, 600, 2000):
        _say(f"[plans] tuned table M={M}: {op.describe(M)}")
        inp = synth.make_inputs(M, SHAPE, seed=70 + M, device="cuda", weights=weights)
        out = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
        torch.cuda.synchronize()
        rows = None if M <= 600 else sample_rows(M)
        check_rows(out, run_oracle(inp, rows), rows)
    op.close()


def test_bad_table_leaves_the_handle_unchanged(H, weights):
    op = H.HCGR(H.Config(), 0)
    good = [{"tokens": 64, "kind": H.HCGR_PLAN_TILE, "down_variant": 0, "streams_per_wg": 1, "segments": 4,
             "up_variant": 0, "ranges": 1}]
    op.set_plan_table(good)
    before = op.describe(64)
    with pytest.raises(H.HcgrError):
        H.hcgr_set_plan_table(op.handle, good + [dict(good[0], tokens=32)])  # keys not increasing
    assert H.hcgr_plan_lookup(op.cfg, good, 64)[1] == before
    inp = synth.make_inputs(64, SHAPE, seed=71, device="cuda", weights=weights)
    out = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    torch.cuda.synchronize()
    check_all(out, run_oracle(inp))
    op.close()


@pytest.mark.parametrize("hc,merged", [(4, False), (4, True), (1, False), (2, False), (8, False)])
def test_shipped_table_at_every_tuned_key(H, weights, hc, merged):
    """Every non-heuristic entry of the shipped tables (HS = 2560, r = 320 at
    every stream count), at its own key, against the oracle (sampled rows
    above 1024 tokens)."""
    cfg = H.Config(weight_layout=H.HCGR_WEIGHTS_MERGED_FOLDED, n_pad=336) if merged else H.Config(hc=hc)
    shape = synth.Shape(hc, 2560, 320)
    op = H.HCGR(cfg, 0, plan_table="shipped")
    assert op.table
    for e in op.table:
        if e["kind"] == H.HCGR_PLAN_HEURISTIC:
            continue
        M = e["tokens"]
        _say(f"[plans] shipped hc={hc} merged={merged} M={M}: {op.describe(M)}")
        inp = synth.make_inputs(M, shape, seed=80 + M, device="cuda", weights=weights if hc == 4 else None)
        wd = synth.fold_merged_weight(inp["wd"], inp["wi"], inp["wnorm"], 336, shape.hs) if merged else inp["wd"]
        out = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], wd, None if merged else inp["wi"], inp["wu"])
        torch.cuda.synchronize()
        rows = None if M <= 1024 else sample_rows(M)
        R, y, inj = inp["R"], inp["y"], inp["inj"]
        if rows is not None:
            idx = torch.as_tensor(rows, device="cuda")
            R, y, inj = R[idx], y[idx], inj[idx]
        ocfg = oracle.OracleConfig(hc=hc, merged=merged, n_pad=336 if merged else 0)
        ref = oracle.forward(ocfg, R.cpu(), y.cpu(), inj.cpu(), inp["wnorm"].cpu(), wd.cpu(),
                             None if merged else inp["wi"].cpu(), inp["wu"].cpu())
        check_rows(out, ref, rows)
    op.close()


def _tile128(M, seg, up, ranges=1):
    import skinny_gemm_hcgr_amd as H
    return {"tokens": M, "kind": H.HCGR_PLAN_TILE, "down_variant": 1, "streams_per_wg": 1, "segments": seg,
            "up_variant": up, "ranges": ranges}


@pytest.mark.parametrize("hc,hs,r,M,seg,up,extra", [
    (4, 2560, 320, 129, 4, 0, ""), (4, 2560, 320, 16400, 1, 1, ""), (4, 640, 64, 1000, 5, 0, ""),
    (4, 1024, 512, 700, 2, 0, ""),          # two row splits of the down rows
    (2, 1024, 320, 300, 8, 2, ""), (8, 512, 96, 257, 1, 2, ""), (1, 2560, 64, 90, 10, 2, ""),
    (4, 1280, 160, 500, 2, 1, "wnfull"), (4, 2560, 320, 384, 1, 0, "merged"), (4, 2560, 320, 200, 2, 0, "mix"),
    # the stream-generic up kernel over 128-token tiles: partial last tiles, a half last k stage
    (2, 1024, 320, 300, 8, 3, ""), (8, 512, 96, 257, 1, 3, ""), (2, 1280, 160, 500, 2, 3, "wnfull"),
    (8, 1024, 320, 1000, 1, 3, "mix"),
])
def test_tile128_shapes(H, hc, hs, r, M, seg, up, extra):
    """The 128-token down tile (two tokens per thread, a prefetch ring of
    three stages, groups of six iterations) across shapes: partial last tiles,
    column segments, row splits, other stream counts, full-width Wnorm, merged
    weights and the mix entry point."""
    shape = synth.Shape(hc=hc, hs=hs, r=r)
    merged = extra == "merged"
    n_pad = (r + hc + 15) // 16 * 16
    cfg = H.Config(hc=hc, hs=hs, r=r, wnorm_len=hc * hs if extra == "wnfull" else 0,
                   weight_layout=H.HCGR_WEIGHTS_MERGED_FOLDED if merged else H.HCGR_WEIGHTS_SEPARATE,
                   n_pad=n_pad if merged else 0)
    op = H.HCGR(cfg, 0, plan_table=[_tile128(M, seg, up)])
    desc = op.describe(M)
    _say(f"[plans] tile128 {extra} hc={hc} hs={hs} r={r} M={M}: {desc}")
    assert "k1_tile tm=128" in desc
    inp = synth.make_inputs(M, shape, seed=90 + M, device="cuda", wnorm_full=extra == "wnfull")
    wd = synth.fold_merged_weight(inp["wd"], inp["wi"], inp["wnorm"], n_pad, hs) if merged else inp["wd"]
    wi = None if merged else inp["wi"]
    ocfg = oracle.OracleConfig(hc=hc, hs=hs, r=r, wnorm_full=extra == "wnfull", merged=merged,
                               n_pad=n_pad if merged else 0)
    rows = None if M <= 1000 else sample_rows(M)
    sel = (lambda t: t) if rows is None else (lambda t: t[torch.as_tensor(rows, device="cuda")])
    if extra == "mix":
        out = op.mix(inp["R"], inp["wnorm"], wd, wi, inp["wu"])
        torch.cuda.synchronize()
        ref = oracle.mix(ocfg, sel(inp["R"]).cpu(), inp["wnorm"].cpu(), wd.cpu(), wi.cpu(), inp["wu"].cpu())
        from parity import check_rrms, check_tol
        check_rrms(sel(out["rrms"]), ref["rrms"])
        check_tol(sel(out["inj_next"]), ref["inj_next"], "inj_next")
        check_tol(sel(out["x"]), ref["x"], "x")
    else:
        out = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], wd, wi, inp["wu"])
        torch.cuda.synchronize()
        ref = oracle.forward(ocfg, sel(inp["R"]).cpu(), sel(inp["y"]).cpu(), sel(inp["inj"]).cpu(),
                             inp["wnorm"].cpu(), wd.cpu(), None if merged else wi.cpu(), inp["wu"].cpu())
        check_rows(out, ref, rows)
    op.close()


@pytest.mark.parametrize("M", [97, 129, 200, 256])
def test_split128_up_tiles(H, weights, M):
    """The decode plan with 128-token down tiles and 32-token up tiles: the up
    grid covers M, not the down kernel's padded count, so a last down tile
    that is mostly padding leaves no up tile wholly past M."""
    table = [{"tokens": M, "kind": H.HCGR_PLAN_SPLIT, "down_variant": 10, "streams_per_wg": 0, "segments": 0,
              "up_variant": 0, "ranges": 0}]
    op = H.HCGR(H.Config(), 0, plan_table=table)
    desc = op.describe(M)
    _say(f"[plans] split128 M={M}: {desc}")
    tiles = (M + 31) // 32  # four 32-token up tiles take 10 channels (256 per tile), more take 16 (160)
    assert "k1_dec tm=128" in desc and "k2_dec tm=32" in desc and f"grid={256 if tiles == 4 else 160}x{tiles}" in desc
    inp = synth.make_inputs(M, SHAPE, seed=700 + M, device="cuda", weights=weights)
    out = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    torch.cuda.synchronize()
    check_rows(out, run_oracle(inp), None)
    op.close()


@pytest.mark.parametrize("hs,r,M,ranges,extra", [
    (2560, 320, 300, 1, ""), (2560, 320, 300, 3, ""),        # a partial second tile; ranges of 27/26 groups
    (2560, 320, 5000, 7, ""), (2560, 320, 65536, 1, ""),     # sampled rows
    (640, 96, 257, 2, ""), (1024, 192, 700, 16, ""),         # two and three k stages; one pair of groups per range
    (1280, 160, 500, 2, "wnfull"), (2560, 320, 1000, 2, "merged"), (2560, 256, 600, 4, "mix"),
    (2560, 320, 100, 4, ""),                                 # one partial tile
    (1024, 288, 600, 4, ""),                                 # last k chunk partly past r
    (2560, 320, 2000, 8, "wnfull"),                          # full-width Wnorm with five k chunks
])
def test_sweep256_shapes(H, hs, r, M, ranges, extra):
    """The up kernel over 256-token tiles (up variant 4): partial last tiles,
    channel ranges down to one pair of 32-channel groups, k stages of 64 with
    a part past r, full-width Wnorm, merged weights and the mix entry point."""
    shape = synth.Shape(hc=4, hs=hs, r=r)
    merged = extra == "merged"
    n_pad = (r + 4 + 15) // 16 * 16
    cfg = H.Config(hs=hs, r=r, wnorm_len=4 * hs if extra == "wnfull" else 0,
                   weight_layout=H.HCGR_WEIGHTS_MERGED_FOLDED if merged else H.HCGR_WEIGHTS_SEPARATE,
                   n_pad=n_pad if merged else 0)
    op = H.HCGR(cfg, 0, plan_table=[_tile128(M, 1, 4, ranges)])
    desc = op.describe(M)
    _say(f"[plans] sweep256 {extra} hs={hs} r={r} M={M} ranges={ranges}: {desc}")
    assert "k2_sweep2" in desc
    inp = synth.make_inputs(M, shape, seed=40 + M, device="cuda", wnorm_full=extra == "wnfull")
    wd = synth.fold_merged_weight(inp["wd"], inp["wi"], inp["wnorm"], n_pad, hs) if merged else inp["wd"]
    wi = None if merged else inp["wi"]
    ocfg = oracle.OracleConfig(hs=hs, r=r, wnorm_full=extra == "wnfull", merged=merged, n_pad=n_pad if merged else 0)
    rows = None if M <= 1000 else sample_rows(M, n=64)
    sel = (lambda t: t) if rows is None else (lambda t: t[torch.as_tensor(rows, device="cuda")])
    if extra == "mix":
        out = op.mix(inp["R"], inp["wnorm"], wd, wi, inp["wu"])
        torch.cuda.synchronize()
        ref = oracle.mix(ocfg, sel(inp["R"]).cpu(), inp["wnorm"].cpu(), wd.cpu(), wi.cpu(), inp["wu"].cpu())
        from parity import check_rrms, check_tol
        check_rrms(sel(out["rrms"]), ref["rrms"])
        check_tol(sel(out["inj_next"]), ref["inj_next"], "inj_next")
        check_tol(sel(out["x"]), ref["x"], "x")
    else:
        out = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], wd, wi, inp["wu"])
        torch.cuda.synchronize()
        ref = oracle.forward(ocfg, sel(inp["R"]).cpu(), sel(inp["y"]).cpu(), sel(inp["inj"]).cpu(),
                             inp["wnorm"].cpu(), wd.cpu(), None if merged else wi.cpu(), inp["wu"].cpu())
        check_rows(out, ref, rows)
    op.close()
