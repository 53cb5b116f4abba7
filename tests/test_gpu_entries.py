"""GPU parity of the combine-only and mix entry points (hcgr_combine,
hcgr_mix, called through the C ABI binding) against the fp64 oracle's
combine and mix, and a layer chain mix -> forward -> forward -> combine that
feeds each call's strided inj_next into the next call."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_r2, check_rrms, check_tol, to64

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
def op(H):
    o = H.HCGR(H.Config(), 0)
    yield o
    o.close()


@pytest.fixture(scope="module")
def weights():
    return synth.make_weights(SHAPE, seed=0, device="cuda")


def _say(msg):
    print(msg, flush=True)


def sample_rows(M, n=64, seed=2):
    rng = np.random.default_rng(seed)
    rows = {0, 1, M // 2, M - 2, M - 1} | set(rng.choice(M, size=min(n, M), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < M))


def oracle_combine(cfg, R, y, inj):
    return oracle.combine(cfg, R.cpu(), y.cpu(), inj.cpu().contiguous(), ld_inj=inj.shape[1])["R2"]


def oracle_mix(cfg, inp, R, wd_key="wd"):
    return oracle.mix(cfg, R.cpu(), inp["wnorm"].cpu(), inp[wd_key].cpu(),
                      None if cfg.merged else inp["wi"].cpu(), inp["wu"].cpu())


def check_mix(out, ref, rows=None):
    sel = (lambda t: t) if rows is None else (lambda t: t[torch.as_tensor(rows, device=t.device)])
    check_rrms(sel(out["rrms"]), ref["rrms"])
    check_tol(sel(out["inj_next"]), ref["inj_next"], "inj_next")
    check_tol(sel(out["x"]), ref["x"], "x")


# ----------------------------------------------------------------- combine --
@pytest.mark.parametrize("M", [1, 2, 7, 8, 9, 32, 33, 100, 1024, 4097])
def test_combine_every_row(op, weights, M):
    _say(f"[entries] combine M={M}")
    inp = synth.make_inputs(M, SHAPE, seed=30, device="cuda", weights=weights)
    R2 = op.combine(inp["R"], inp["y"], inp["inj"])
    torch.cuda.synchronize()
    check_r2(R2, oracle_combine(oracle.OracleConfig(), inp["R"], inp["y"], inp["inj"]))


@pytest.mark.parametrize("M", [8192, 65536])
def test_combine_large_sampled_rows(op, weights, M):
    """The large-M workloads, in the configuration the benchmark times (oracle
    on sampled rows; every row is independent)."""
    _say(f"[entries] combine sampled M={M}")
    inp = synth.make_inputs(M, SHAPE, seed=0, device="cuda", weights=weights)
    R2 = op.combine(inp["R"], inp["y"], inp["inj"])
    torch.cuda.synchronize()
    rows = sample_rows(M)
    idx = torch.as_tensor(rows, device="cuda")
    check_r2(R2[idx], oracle_combine(oracle.OracleConfig(), inp["R"][idx], inp["y"][idx], inp["inj"][idx]))


@pytest.mark.parametrize("hs,M", [(128, 50), (640, 17), (8192, 9), (24576, 3), (65536, 2)])
def test_combine_shapes(H, hs, M):
    """Stream widths from one 16-byte chunk per thread (HS = 128, most threads
    idle) up to several passes per row (HS = 24576 and 65536)."""
    _say(f"[entries] combine hs={hs} M={M}")
    shape = synth.Shape(hs=hs, r=32)
    o = H.HCGR(H.Config(hs=hs, r=32), 0)
    inp = synth.make_inputs(M, shape, seed=31, device="cuda")
    R2 = o.combine(inp["R"], inp["y"], inp["inj"])
    torch.cuda.synchronize()
    check_r2(R2, oracle_combine(oracle.OracleConfig(hs=hs, r=32), inp["R"], inp["y"], inp["inj"]))
    o.close()


def test_combine_matches_forward_r2_bitwise(op, weights):
    """The combine entry point and the whole op form R2 with the same
    arithmetic: identical bits."""
    for M in (5, 64, 3000):
        inp = synth.make_inputs(M, SHAPE, seed=32, device="cuda", weights=weights)
        R2 = op.combine(inp["R"], inp["y"], inp["inj"])
        full = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
        torch.cuda.synchronize()
        assert torch.equal(R2, full["R2"]), M


def test_combine_strided_logits_and_cancellation(op, weights):
    """Logits in a strided [M, 336] view (padding 1000 that must not be read),
    and R = -bf16(y*iw) so that R2 nearly cancels: still within one ulp."""
    M = 40
    inp = synth.make_inputs(M, SHAPE, seed=33, device="cuda", weights=weights, ld_inj=336)
    assert inp["inj"].shape == (M, 336)
    inp["inj"][:, SHAPE.hc:] = 1000.0
    iw = 2.0 / (1.0 + torch.exp(-inp["inj"][:, :SHAPE.hc].double().cpu() / SHAPE.hc))
    y = inp["y"].double().cpu()
    R = -(y[:, None, :] * iw[:, :, None]).reshape(M, SHAPE.k)
    R[M // 2:] = inp["R"][M // 2:].double().cpu()  # half the rows without cancellation
    inp["R"] = R.to(torch.bfloat16).cuda()
    R2 = op.combine(inp["R"], inp["y"], inp["inj"])
    torch.cuda.synchronize()
    check_r2(R2, oracle_combine(oracle.OracleConfig(), inp["R"], inp["y"], inp["inj"]))


def test_combine_m0_and_errors(H, op, weights):
    assert H.hcgr_combine(op.handle, None, None, None, 4, 0, None) == H.HCGR_OK
    inp = synth.make_inputs(4, SHAPE, seed=34, device="cuda", weights=weights)
    keep = inp["R"].clone()
    with pytest.raises(H.HcgrError) as e:  # in place: R2 aliases R
        H.hcgr_combine(op.handle, inp["R"], inp["y"], inp["inj"], 4, 4, inp["R"])
    assert e.value.status == H.HCGR_ERR_ALIASING
    torch.cuda.synchronize()
    assert torch.equal(keep, inp["R"])


# --------------------------------------------------------------------- mix --
@pytest.mark.parametrize("M", [1, 5, 16, 32, 64, 65, 129, 300, 1024])
def test_mix_every_row(op, weights, M):
    _say(f"[entries] mix M={M} plan: {__import__('skinny_gemm_hcgr_amd').hcgr_describe_plan(op.cfg, M)}")
    inp = synth.make_inputs(M, SHAPE, seed=40, device="cuda", weights=weights)
    out = op.mix(inp["R"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    torch.cuda.synchronize()
    check_mix(out, oracle_mix(oracle.OracleConfig(), inp, inp["R"]))


@pytest.mark.parametrize("M", [4096, 8192, 65536])
def test_mix_large_sampled_rows(op, weights, M):
    _say(f"[entries] mix sampled M={M}")
    inp = synth.make_inputs(M, SHAPE, seed=0, device="cuda", weights=weights)
    out = op.mix(inp["R"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    torch.cuda.synchronize()
    rows = sample_rows(M)
    idx = torch.as_tensor(rows, device="cuda")
    check_mix(out, oracle_mix(oracle.OracleConfig(), inp, inp["R"][idx]), rows)


@pytest.mark.parametrize("M", [7, 1024])
def test_mix_merged_folded(H, weights, M):
    o = H.HCGR(H.Config(weight_layout=H.HCGR_WEIGHTS_MERGED_FOLDED, n_pad=336), 0)
    inp = synth.make_inputs(M, SHAPE, seed=41, device="cuda", weights=weights)
    inp["wm"] = synth.fold_merged_weight(inp["wd"], inp["wi"], inp["wnorm"], 336, SHAPE.hs)
    out = o.mix(inp["R"], inp["wnorm"], inp["wm"], None, inp["wu"])
    torch.cuda.synchronize()
    check_mix(out, oracle_mix(oracle.OracleConfig(merged=True, n_pad=336), inp, inp["R"], wd_key="wm"))
    o.close()


@pytest.mark.parametrize("hs,r,M", [(4352, 64, 20), (4224, 64, 8), (640, 64, 8192)])
def test_mix_other_plans(H, hs, r, M):
    """The one- and four-stream fallback down kernels and a column-segmented
    tile plan, each without injection."""
    shape = synth.Shape(hs=hs, r=r)
    o = H.HCGR(H.Config(hs=hs, r=r), 0)
    _say(f"[entries] mix hs={hs} r={r} M={M}: {H.hcgr_describe_plan(o.cfg, M)}")
    inp = synth.make_inputs(M, shape, seed=42, device="cuda")
    out = o.mix(inp["R"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    torch.cuda.synchronize()
    rows = sample_rows(M, 32) if M > 64 else None
    R = inp["R"] if rows is None else inp["R"][torch.as_tensor(rows, device="cuda")]
    check_mix(out, oracle_mix(oracle.OracleConfig(hs=hs, r=r), inp, R), rows)
    o.close()


def test_mix_equals_forward_with_zero_block_output(op, weights):
    """mix(R) is the whole op with y = 0 (then R2 = R whatever the logits):
    rrms, inj_next and x bit for bit, at decode and tile sizes."""
    for M in (3, 32, 2048):
        inp = synth.make_inputs(M, SHAPE, seed=43, device="cuda", weights=weights)
        m = op.mix(inp["R"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
        f = op.forward(inp["R"], torch.zeros_like(inp["y"]), inp["inj"], inp["wnorm"], inp["wd"], inp["wi"],
                       inp["wu"])
        torch.cuda.synchronize()
        assert torch.equal(f["R2"], inp["R"])
        for k in ("rrms", "inj_next", "x"):
            assert torch.equal(m[k], f[k]), (M, k)


def test_mix_graph_replay(op, weights):
    M = 32
    inp = synth.make_inputs(M, SHAPE, seed=44, device="cuda", weights=weights)
    out = op.alloc_outputs(M)
    ws = op.workspace(M)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        op.mix(inp["R"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        op.mix(inp["R"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], out=out, workspace=ws)
    for rep in range(3):
        fresh = synth.make_inputs(M, SHAPE, seed=140 + rep, device="cuda", weights=weights)
        inp["R"].copy_(fresh["R"])
        g.replay()
        torch.cuda.synchronize()
        eager = op.mix(fresh["R"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
        torch.cuda.synchronize()
        for k in ("rrms", "inj_next", "x"):
            assert torch.equal(out[k], eager[k]), (rep, k)
        if rep == 0:
            check_mix(out, oracle_mix(oracle.OracleConfig(), inp, fresh["R"]))


def test_mix_errors_on_device(H, op, weights):
    inp = synth.make_inputs(4, SHAPE, seed=45, device="cuda", weights=weights)
    out = op.alloc_outputs(4)
    ws = op.workspace(4)
    with pytest.raises(H.HcgrError) as e:  # x written over the residual input
        H.hcgr_mix(op.handle, inp["R"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], 4, out["rrms"],
                   out["inj_next"], 4, inp["R"], ws, ws.numel())
    assert e.value.status == H.HCGR_ERR_ALIASING


# ------------------------------------------------------------- layer chain --
def test_layer_chain(op, weights):
    """Four layers: mix (first layer, no block output yet) -> forward ->
    forward -> combine (last layer, no mixed input needed). Every call's
    inj_next goes to a packed [M, 336] buffer (row stride 336) and is fed to
    the next call as its strided logits; each GPU call is checked against the
    oracle on the very inputs it received."""
    M = 48
    cfg = oracle.OracleConfig()
    inp = synth.make_inputs(M, SHAPE, seed=50, device="cuda", weights=weights)
    R = inp["R"]
    out0 = op.alloc_outputs(M, 336)
    op.mix(R, inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], out=out0)
    torch.cuda.synchronize()
    check_mix(out0, oracle_mix(cfg, inp, R))
    assert torch.all(out0["inj_next_buf"][:, SHAPE.hc:] == 0)
    inj = out0["inj_next"]
    for layer in (1, 2):
        y = synth.normal_bf16(60 + layer, 2, M, SHAPE.hs, device="cuda")  # the block's output
        out = op.alloc_outputs(M, 336)
        op.forward(R, y, inj, inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], out=out)
        torch.cuda.synchronize()
        ref = oracle.forward(cfg, R.cpu(), y.cpu(), inj.cpu().contiguous(), inp["wnorm"].cpu(), inp["wd"].cpu(),
                             inp["wi"].cpu(), inp["wu"].cpu())
        check_r2(out["R2"], ref["R2"])
        check_mix(out, ref)
        R, inj = out["R2"], out["inj_next"]
    y = synth.normal_bf16(63, 2, M, SHAPE.hs, device="cuda")
    R_last = op.combine(R, y, inj)
    torch.cuda.synchronize()
    check_r2(R_last, oracle_combine(cfg, R, y, inj))
