"""GPU parity of the decode plans whose chunk reduction is done by the last
workgroup to arrive at a per-block counter: the fused plan (down kernel + up
kernel; the heuristic at decode sizes with one or two streams) and the
persistent plan (one kernel whose up-role workgroups wait for the down role's
h), against the fp64 oracle at every stream count, with the merged/folded
layout, full-width Wnorm, wide gates, the mix entry point, graph replay and a
long interleaved run on one workspace. After every call the workspace's
counter bytes must be back at zero, including the persistent plan's
gave-up word."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_all, check_rrms, check_tol

pytestmark = pytest.mark.gpu

FUSED, PERSISTENT = 4, 5


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import skinny_gemm_hcgr_amd as H
    H.load_library()
    return H


def _say(msg):
    print(msg, flush=True)


def table(kind, M):
    return [{"tokens": M, "kind": kind, "down_variant": int(M > 16)}]


def make_op(H, kind, M, cfg=None):
    op = H.HCGR(cfg or H.Config(), 0, plan_table=table(kind, M))
    assert op.describe(M).startswith(f"M={M} plan={'fused' if kind == FUSED else 'persistent'}"), op.describe(M)
    return op


def counters_clear(H, ws):
    c = ws[:H.HCGR_WORKSPACE_COUNTER_BYTES]
    assert int(c.count_nonzero()) == 0, c.view(torch.int32).nonzero().flatten().tolist()


def oracle_forward(cfg, inp, wd_key="wd"):
    return oracle.forward(cfg, inp["R"].cpu(), inp["y"].cpu(), inp["inj"].cpu().contiguous(), inp["wnorm"].cpu(),
                          inp[wd_key].cpu(), None if cfg.merged else inp["wi"].cpu(), inp["wu"].cpu(),
                          ld_inj=inp["inj"].shape[1])


CASES = [(kind, hc, M) for kind in (FUSED, PERSISTENT) for hc in (1, 2, 4, 8)
         for M in (1, 5, 16, 17, 31, 32, 33, 64, 100)]


@pytest.mark.parametrize("kind,hc,M", CASES)
def test_decode_plans_every_row(H, kind, hc, M):
    """Every row at every stream count, token tiles of 16 and 32 with ragged
    tails and up to four tiles (each with its own counters)."""
    cfg = H.Config(hc=hc)
    op = make_op(H, kind, M, cfg)
    _say(f"[decode] {op.describe(M)[:110]}")
    inp = synth.make_inputs(M, synth.Shape(hc, 2560, 320), seed=31 + M, device="cuda")
    out = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    torch.cuda.synchronize()
    check_all(out, oracle_forward(oracle.OracleConfig(hc=hc), inp))
    counters_clear(H, op._ws)
    op.close()


@pytest.mark.parametrize("kind", [FUSED, PERSISTENT])
@pytest.mark.parametrize("hc,hs,r,M", [(4, 384, 96, 7), (1, 8192, 64, 20), (2, 1024, 512, 32), (8, 640, 320, 3),
                                      (4, 1280, 128, 18)])
def test_decode_plans_other_shapes(H, kind, hc, hs, r, M):
    """Other widths and ranks: one-unit chunks (HS = 384), a wide stream split
    into chunks of unequal width (HS = 8192 in 28 chunks), the widest rank,
    a narrow stream with eight streams, and HS = 1280 (chunks of 3 and 2
    units)."""
    cfg = H.Config(hc=hc, hs=hs, r=r)
    op = make_op(H, kind, M, cfg)
    _say(f"[decode] hc={hc} hs={hs} r={r} {op.describe(M)[:100]}")
    inp = synth.make_inputs(M, synth.Shape(hc, hs, r), seed=5, device="cuda")
    out = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    torch.cuda.synchronize()
    check_all(out, oracle_forward(oracle.OracleConfig(hc=hc, hs=hs, r=r), inp))
    counters_clear(H, op._ws)
    op.close()


@pytest.mark.parametrize("kind", [FUSED, PERSISTENT])
@pytest.mark.parametrize("M", [1, 32])
def test_decode_plans_merged_folded(H, kind, M):
    """The merged 336-row weight with (1 + Wnorm) folded into its columns."""
    cfg = H.Config(weight_layout=H.HCGR_WEIGHTS_MERGED_FOLDED, n_pad=336)
    op = make_op(H, kind, M, cfg)
    inp = synth.make_inputs(M, synth.Shape(), seed=8, device="cuda")
    inp["wm"] = synth.fold_merged_weight(inp["wd"], inp["wi"], inp["wnorm"], 336, 2560)
    out = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wm"], None, inp["wu"])
    torch.cuda.synchronize()
    check_all(out, oracle_forward(oracle.OracleConfig(merged=True, n_pad=336), inp, wd_key="wm"))
    counters_clear(H, op._ws)
    op.close()


@pytest.mark.parametrize("kind", [FUSED, PERSISTENT])
@pytest.mark.parametrize("hc", [2, 4])
def test_decode_plans_full_width_wnorm_and_wide_gates(H, kind, hc):
    """Wnorm indexed by k, and projections wide enough that the gate spans
    (0, 1), with a strided inj_next."""
    M = 24
    cfg = H.Config(hc=hc, wnorm_len=hc * 2560)
    op = make_op(H, kind, M, cfg)
    sh = synth.Shape(hc, 2560, 320)
    inp = synth.make_inputs(M, sh, seed=9, device="cuda", wnorm_full=True, wd_std=8 / np.sqrt(sh.k),
                            wu_std=2 / np.sqrt(320), ld_inj=hc + 3)
    out = op.alloc_outputs(M, ld_inj_next=hc + 5)
    op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], out=out)
    torch.cuda.synchronize()
    check_all(out, oracle_forward(oracle.OracleConfig(hc=hc, wnorm_full=True), inp))
    assert int(out["inj_next_buf"][:, hc:].count_nonzero()) == 0  # columns past HC untouched
    counters_clear(H, op._ws)
    op.close()


@pytest.mark.parametrize("kind", [FUSED, PERSISTENT])
def test_decode_plans_mix_entry(H, kind):
    """The mix entry point (R taken as R2: no y, no logits, no R2 output)."""
    M = 9
    op = make_op(H, kind, M)
    inp = synth.make_inputs(M, synth.Shape(), seed=12, device="cuda")
    out = op.mix(inp["R"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    torch.cuda.synchronize()
    ref = oracle.mix(oracle.OracleConfig(), inp["R"].cpu(), inp["wnorm"].cpu(), inp["wd"].cpu(), inp["wi"].cpu(),
                     inp["wu"].cpu())
    check_rrms(out["rrms"], ref["rrms"])
    check_tol(out["inj_next"], ref["inj_next"], "inj_next")
    check_tol(out["x"], ref["x"], "x")
    counters_clear(H, op._ws)
    op.close()


@pytest.mark.parametrize("kind", [FUSED, PERSISTENT])
def test_decode_plans_graph_replay(H, kind):
    """Calls captured into a HIP graph and replayed with new inputs and eager
    work in between: every replay bitwise equal to an eager call of the same
    plan, the counters back at zero after each."""
    M = 20
    op = make_op(H, kind, M)
    w = synth.make_weights(synth.Shape(), seed=0, device="cuda")
    inp = synth.make_inputs(M, synth.Shape(), seed=40, device="cuda", weights=w)
    out = op.alloc_outputs(M)
    ws = op.workspace(M)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], out=out, workspace=ws)
    eager_ws = H.new_workspace(H.hcgr_workspace_size(op.handle, M))
    for rep in range(4):
        fresh = synth.make_inputs(M, synth.Shape(), seed=50 + rep, device="cuda", weights=w)
        for k in ("R", "y", "inj"):
            inp[k].copy_(fresh[k])
        g.replay()
        torch.cuda.synchronize()
        counters_clear(H, ws)
        eager = op.forward(fresh["R"], fresh["y"], fresh["inj"], fresh["wnorm"], fresh["wd"], fresh["wi"],
                           fresh["wu"], workspace=eager_ws)
        torch.cuda.synchronize()
        for k in ("R2", "rrms", "inj_next", "x"):
            assert torch.equal(out[k], eager[k]), (rep, k)
        if rep == 0:
            check_all(out, oracle_forward(oracle.OracleConfig(), fresh))
    del g
    op.close()


@pytest.mark.parametrize("kind", [FUSED, PERSISTENT])
def test_decode_plans_interleaved_stress(H, kind):
    """Many back-to-back calls of four sizes (one to three token tiles)
    interleaved on one workspace without synchronisation: bitwise identical
    results every time, matching the oracle, counters zero at the end."""
    sizes = (5, 32, 70, 1)
    ops = {M: make_op(H, kind, M) for M in sizes}
    ws = H.new_workspace(max(H.hcgr_workspace_size(ops[M].handle, M) for M in sizes))
    w = synth.make_weights(synth.Shape(), seed=0, device="cuda")
    inps = {M: synth.make_inputs(M, synth.Shape(), seed=60 + M, device="cuda", weights=w) for M in sizes}
    outs = {M: ops[M].alloc_outputs(M) for M in sizes}
    first = {}
    for rep in range(25):
        for M in sizes:
            inp = inps[M]
            ops[M].forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"],
                           out=outs[M], workspace=ws)
            if rep == 0:
                torch.cuda.synchronize()
                first[M] = {k: outs[M][k].clone() for k in ("R2", "rrms", "inj_next", "x")}
            elif rep % 6 == 0 or rep == 24:
                torch.cuda.synchronize()
                for k in first[M]:
                    assert torch.equal(first[M][k], outs[M][k]), (rep, M, k)
    torch.cuda.synchronize()
    counters_clear(H, ws)
    for M in sizes:
        check_all(outs[M], oracle_forward(oracle.OracleConfig(), inps[M]))
        ops[M].close()


def test_persistent_wait_that_gives_up(H):
    """The persistent plan's bounded wait, forced from the host to give up at
    once (a poll budget of 0): the launch completes, the workspace's error
    counter reads 1, and once the caller has zeroed the counter bytes and
    restored the budget, the next call on the same workspace matches the
    oracle and leaves every counter at zero. Budgets outside 0..2^24 are
    rejected."""
    M = 5
    op = make_op(H, PERSISTENT, M)
    for bad in (-1, H.HCGR_MAX_WAIT_POLLS + 1):
        with pytest.raises(H.HcgrError):
            op.set_wait_polls(bad)
    inp = synth.make_inputs(M, synth.Shape(), seed=77, device="cuda")
    ws = op.workspace(M)
    op.set_wait_polls(0)
    _say("[decode] persistent M=5 with a poll budget of 0")
    op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], workspace=ws)
    torch.cuda.synchronize()
    n = H.HCGR_WORKSPACE_COUNTER_BYTES
    assert int(ws[n - 128:n - 124].view(torch.int32)[0]) == 1
    ws[:n].zero_()
    op.set_wait_polls(H.HCGR_DEFAULT_WAIT_POLLS)
    out = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], workspace=ws)
    torch.cuda.synchronize()
    check_all(out, oracle_forward(oracle.OracleConfig(), inp))
    counters_clear(H, ws)
    op.close()


@pytest.mark.parametrize("hc", [1, 2, 8])
@pytest.mark.parametrize("kd", list(range(11)))
def test_split_plan_other_stream_counts(H, hc, kd):
    """The split plan at HC = 1, 2, 8 (the reduction over HC streams, the
    stream-generic decode up kernel over 16-, 32- and 64-token tiles): every
    down-kernel variant, every row, at a ragged token count and one past a
    token tile."""
    cfg = H.Config(hc=hc)
    for M in (3, 33):
        op = H.HCGR(cfg, 0, plan_table=[{"tokens": M, "kind": 0, "down_variant": kd}])
        d = op.describe(M)
        if "plan=split" not in d:  # this variant cannot split the stream width
            op.close()
            continue
        _say(f"[split] hc={hc} {d[:100]}")
        inp = synth.make_inputs(M, synth.Shape(hc, 2560, 320), seed=kd + M, device="cuda")
        out = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
        torch.cuda.synchronize()
        check_all(out, oracle_forward(oracle.OracleConfig(hc=hc), inp))
        op.close()


def test_split_is_the_decode_heuristic_for_other_stream_counts(H):
    """The heuristic plan at decode sizes with HC = 1, 2, 8 is the split plan
    with the stream-generic kernels, matching the oracle."""
    for hc, M in ((1, 32), (2, 3), (8, 17)):
        cfg = H.Config(hc=hc)
        assert "plan=split" in H.hcgr_describe_plan(cfg, M)
        op = H.HCGR(cfg, 0)
        inp = synth.make_inputs(M, synth.Shape(hc, 2560, 320), seed=70, device="cuda")
        out = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
        torch.cuda.synchronize()
        check_all(out, oracle_forward(oracle.OracleConfig(hc=hc), inp))
        counters_clear(H, op._ws)
        op.close()
