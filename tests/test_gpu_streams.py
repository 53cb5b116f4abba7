"""GPU parity at stream counts other than 4 (HC = 1, 2, 8): the tile plan at
every M with one stream per down workgroup, the stream sum over HC partials
and the HC-generic up kernel, against the fp64 oracle (which is generic in
HC); plus the merged layout, full-width Wnorm, the combine and mix entry
points, strided chaining and graph replay at these stream counts."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_all, check_r2, check_rrms, check_tol

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import skinny_gemm_hcgr_amd as H
    H.load_library()
    return H


def _say(msg):
    print(msg, flush=True)


def sample_rows(M, n=24, seed=5):
    rng = np.random.default_rng(seed)
    rows = {0, 1, M // 2, M - 2, M - 1} | set(rng.choice(M, size=min(n, M), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < M))


def sel(t, rows):
    return t if rows is None else t[torch.as_tensor(rows, device=t.device)]


def oracle_forward(cfg, inp, rows=None, wd_key="wd"):
    R, y, inj = sel(inp["R"], rows), sel(inp["y"], rows), sel(inp["inj"], rows)
    return oracle.forward(cfg, R.cpu(), y.cpu(), inj.cpu().contiguous(), inp["wnorm"].cpu(), inp[wd_key].cpu(),
                          None if cfg.merged else inp["wi"].cpu(), inp["wu"].cpu(), ld_inj=inj.shape[1])


def check_rows(out, ref, rows):
    check_all({k: sel(out[k], rows) for k in ("R2", "rrms", "inj_next", "x")}, ref)


CASES = [(hc, hs, r, M) for hc in (1, 2, 8) for hs, r in ((2560, 320), (384, 96), (1024, 512))
         for M in (1, 33, 130, 2100)]


@pytest.mark.parametrize("hc,hs,r,M", CASES)
def test_stream_counts(H, hc, hs, r, M):
    shape = synth.Shape(hc=hc, hs=hs, r=r)
    o = H.HCGR(H.Config(hc=hc, hs=hs, r=r), 0)
    _say(f"[streams] hc={hc} hs={hs} r={r} M={M}: {H.hcgr_describe_plan(o.cfg, M)}")
    inp = synth.make_inputs(M, shape, seed=70 + hc + M, device="cuda")
    out = o.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    torch.cuda.synchronize()
    rows = None if M <= 130 else sample_rows(M)
    check_rows(out, oracle_forward(oracle.OracleConfig(hc=hc, hs=hs, r=r), inp, rows), rows)
    o.close()


@pytest.mark.parametrize("hc,M", [(2, 5), (2, 500), (8, 70)])
def test_stream_counts_merged_folded(H, hc, M):
    hs, r, n_pad = 1024, 320, 336
    shape = synth.Shape(hc=hc, hs=hs, r=r)
    o = H.HCGR(H.Config(hc=hc, hs=hs, r=r, weight_layout=H.HCGR_WEIGHTS_MERGED_FOLDED, n_pad=n_pad), 0)
    inp = synth.make_inputs(M, shape, seed=80 + M, device="cuda")
    inp["wm"] = synth.fold_merged_weight(inp["wd"], inp["wi"], inp["wnorm"], n_pad, hs)
    out = o.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wm"], None, inp["wu"])
    torch.cuda.synchronize()
    rows = None if M <= 130 else sample_rows(M)
    cfg = oracle.OracleConfig(hc=hc, hs=hs, r=r, merged=True, n_pad=n_pad)
    check_rows(out, oracle_forward(cfg, inp, rows, wd_key="wm"), rows)
    o.close()


@pytest.mark.parametrize("kind", [None, 4])
@pytest.mark.parametrize("full", [False, True])
@pytest.mark.parametrize("M", [1, 17, 32])
def test_hc8_ten_channel_up_kernel(H, kind, full, M):
    """HC = 8 at HS = 2560: the decode up kernel runs five waves of two
    channels (10 channels per workgroup, 256 workgroups), whose R2 rows and
    Wnorm arrive in 4-byte pieces; split plan (heuristic) and fused plan, Wnorm
    per channel or per element, 16- and 32-token tiles; every row against the
    oracle."""
    hs, r = 2560, 320
    _say(f"[streams] hc=8 ten-channel up kernel M={M} full={full} kind={kind}")
    cfg = H.Config(hc=8, hs=hs, r=r, wnorm_len=8 * hs if full else 0)
    o = H.HCGR(cfg, 0, plan_table=[] if kind is None else [{"tokens": M, "kind": kind, "down_variant": int(M > 16)}])
    assert "waves=5 channels=10 grid=256" in o.describe(M), o.describe(M)
    inp = synth.make_inputs(M, synth.Shape(hc=8, hs=hs, r=r), seed=120 + M, device="cuda", wnorm_full=full)
    out = o.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    torch.cuda.synchronize()
    check_all(out, oracle_forward(oracle.OracleConfig(hc=8, hs=hs, r=r, wnorm_full=full), inp))
    o.close()


@pytest.mark.parametrize("full", [False, True])
@pytest.mark.parametrize("hs,M,kd,cw", [(2560, 1, 0, 10), (2560, 17, 4, 10), (2560, 64, 8, 10), (2560, 45, 8, 10),
                                        (2560, 30, 0, 10), (5120, 9, 1, 10), (2560, 90, 4, 16), (2560, 128, 4, 10),
                                        (2560, 150, 4, 16), (2560, 150, 8, 10), (2560, 256, 8, 10), (1280, 30, 4, 16),
                                        (1280, 64, 8, 16)])
def test_hc4_up_kernel_channel_groups(H, full, hs, M, kd, cw):
    """HC = 4 decode up kernel: 10 channels per workgroup (three waves, the
    last one's rows past the tenth channel zero, R2 rows and Wnorm in 4-byte
    pieces) where HS is a multiple of 2560 unless that takes more rounds of
    workgroups than 16 channels, else 16 (four waves: HS = 2560 in three or
    five 32-token tiles, HS = 1280); 16-, 32- and 64-token tiles, one to four
    of them, a ragged last tile, Wnorm per channel or per element; every row
    against the oracle."""
    r = 320
    _say(f"[streams] hc=4 up kernel hs={hs} M={M} kd={kd} full={full}")
    table = [{"tokens": M, "kind": H.HCGR_PLAN_SPLIT, "down_variant": kd, "streams_per_wg": 0, "segments": 0,
              "up_variant": 0, "ranges": 0}]
    o = H.HCGR(H.Config(hc=4, hs=hs, r=r, wnorm_len=4 * hs if full else 0), 0, plan_table=table)
    desc = o.describe(M)
    assert f"k2_dec tm={(16, 32, 64)[kd // 4]} waves={(cw + 3) // 4} channels={cw} grid={hs // cw}x" in desc, desc
    inp = synth.make_inputs(M, synth.Shape(hc=4, hs=hs, r=r), seed=140 + M, device="cuda", wnorm_full=full)
    out = o.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    torch.cuda.synchronize()
    check_all(out, oracle_forward(oracle.OracleConfig(hc=4, hs=hs, r=r, wnorm_full=full), inp))
    o.close()


@pytest.mark.parametrize("hc", [2, 8])
def test_stream_counts_full_width_wnorm(H, hc):
    hs, r, M = 512, 160, 40
    shape = synth.Shape(hc=hc, hs=hs, r=r)
    o = H.HCGR(H.Config(hc=hc, hs=hs, r=r, wnorm_len=hc * hs), 0)
    inp = synth.make_inputs(M, shape, seed=90, device="cuda", wnorm_full=True)
    out = o.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    torch.cuda.synchronize()
    check_all(out, oracle_forward(oracle.OracleConfig(hc=hc, hs=hs, r=r, wnorm_full=True), inp))
    o.close()


@pytest.mark.parametrize("hc", [1, 2, 8])
def test_stream_counts_wide_gates(H, hc):
    """Wider projections so that the gate spans (0, 1) and the HC-generic up
    kernel's sigmoid and MIX carry real weight."""
    hs, r, M = 640, 128, 50
    shape = synth.Shape(hc=hc, hs=hs, r=r)
    o = H.HCGR(H.Config(hc=hc, hs=hs, r=r), 0)
    inp = synth.make_inputs(M, shape, seed=91, device="cuda", wd_std=8 / (hc * hs) ** 0.5, wu_std=2 / r ** 0.5)
    ref = oracle.forward(oracle.OracleConfig(hc=hc, hs=hs, r=r), inp["R"].cpu(), inp["y"].cpu(), inp["inj"].cpu(),
                         inp["wnorm"].cpu(), inp["wd"].cpu(), inp["wi"].cpu(), inp["wu"].cpu(), debug=True)
    assert np.ptp(ref["G"]) > 0.8
    out = o.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    torch.cuda.synchronize()
    check_all(out, ref)
    o.close()


@pytest.mark.parametrize("hc,M", [(1, 5), (2, 100), (8, 37)])
def test_stream_counts_combine_and_mix(H, hc, M):
    hs, r = 768, 96
    shape = synth.Shape(hc=hc, hs=hs, r=r)
    cfg = oracle.OracleConfig(hc=hc, hs=hs, r=r)
    o = H.HCGR(H.Config(hc=hc, hs=hs, r=r), 0)
    inp = synth.make_inputs(M, shape, seed=92, device="cuda")
    R2 = o.combine(inp["R"], inp["y"], inp["inj"])
    mx = o.mix(inp["R"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    torch.cuda.synchronize()
    check_r2(R2, oracle.combine(cfg, inp["R"].cpu(), inp["y"].cpu(), inp["inj"].cpu())["R2"])
    ref = oracle.mix(cfg, inp["R"].cpu(), inp["wnorm"].cpu(), inp["wd"].cpu(), inp["wi"].cpu(), inp["wu"].cpu())
    check_rrms(mx["rrms"], ref["rrms"])
    check_tol(mx["inj_next"], ref["inj_next"], "inj_next")
    check_tol(mx["x"], ref["x"], "x")
    o.close()


@pytest.mark.parametrize("hc", [2, 8])
def test_stream_counts_chain_and_graph(H, hc):
    """inj_next into a packed [M, 64] buffer fed to the next call as strided
    logits, then the same call captured into a HIP graph and replayed with
    new inputs (bitwise equal to eager)."""
    hs, r, M = 512, 64, 48
    shape = synth.Shape(hc=hc, hs=hs, r=r)
    cfg = oracle.OracleConfig(hc=hc, hs=hs, r=r)
    o = H.HCGR(H.Config(hc=hc, hs=hs, r=r), 0)
    inp = synth.make_inputs(M, shape, seed=93, device="cuda")
    out1 = o.alloc_outputs(M, 64)
    o.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], out=out1)
    torch.cuda.synchronize()
    check_all(out1, oracle_forward(cfg, inp))
    assert torch.all(out1["inj_next_buf"][:, hc:] == 0)
    inp2 = dict(inp, R=out1["R2"], y=synth.normal_bf16(94, 2, M, hs, device="cuda"), inj=out1["inj_next"])
    out2 = o.alloc_outputs(M)
    ws = o.workspace(M)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o.forward(inp2["R"], inp2["y"], inp2["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], out=out2,
                  workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    check_all(out2, oracle_forward(cfg, inp2))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        o.forward(inp2["R"], inp2["y"], inp2["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], out=out2,
                  workspace=ws)
    for rep in range(3):
        fresh = synth.make_inputs(M, shape, seed=200 + rep, device="cuda")
        inp2["R"].copy_(fresh["R"])
        inp2["y"].copy_(fresh["y"])
        g.replay()
        torch.cuda.synchronize()
        eager = o.forward(inp2["R"], inp2["y"], inp2["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
        torch.cuda.synchronize()
        for k in ("R2", "rrms", "inj_next", "x"):
            assert torch.equal(out2[k], eager[k]), (rep, k)
    o.close()
