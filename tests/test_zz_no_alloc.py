"""hcgr_forward_noalloc (the entry point that allocates nothing: its workspace
is the library's static per-GPU scratch) against hcgr_forward with a caller
workspace, through the C ABI: bitwise-equal outputs on two calls in a row,
the second smaller and on another plan, plus a decode call on the fused plan
(whose counters live in the scratch), and the size limit rejected on the
host before any launch."""
from __future__ import annotations

import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def H():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import skinny_gemm_hcgr_amd as H
    H.load_library()
    return H


def _call_both(H, op, inp, M):
    ref = op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"])
    out = op.alloc_outputs(M)
    H.hcgr_forward_noalloc(op.handle, inp["R"], inp["y"], inp["inj"], inp["inj"].stride(0), inp["wnorm"], inp["wd"],
                           inp["wi"], inp["wu"], M, out["R2"], out["rrms"], out["inj_next"], out["ld_inj_next"],
                           out["x"])
    torch.cuda.synchronize()
    return ref, out


@pytest.mark.parametrize("hc,sizes", [(4, (2048, 32, 1)), (2, (700, 5))])
def test_noalloc_matches_forward(H, hc, sizes):
    """Calls in a row on the scratch, each smaller than the one before (tile
    plan, then the decode plans), bitwise equal to hcgr_forward."""
    cfg = H.Config(hc=hc)
    op = H.HCGR(cfg, 0)
    w = synth.make_weights(synth.Shape(hc, 2560, 320), seed=0, device="cuda")
    for i, M in enumerate(sizes):
        print(f"[noalloc] hc={hc} M={M} {H.hcgr_describe_plan(cfg, M)[:70]}", flush=True)
        inp = synth.make_inputs(M, synth.Shape(hc, 2560, 320), seed=80 + i, device="cuda", weights=w)
        ref, out = _call_both(H, op, inp, M)
        for k in ("R2", "rrms", "inj_next", "x"):
            assert torch.equal(ref[k], out[k]), (M, k)
    op.close()


def test_noalloc_fused_and_persistent_plans(H):
    """The decode plans whose counters live in the scratch: two calls each,
    bitwise equal to hcgr_forward (the counters must return to zero for the
    second call to be right)."""
    for kind in (H.HCGR_PLAN_FUSED, H.HCGR_PLAN_PERSISTENT):
        op = H.HCGR(H.Config(), 0, plan_table=[{"tokens": 32, "kind": kind, "down_variant": 1}])
        w = synth.make_weights(synth.Shape(), seed=0, device="cuda")
        for M in (32, 19):
            inp = synth.make_inputs(M, synth.Shape(), seed=90 + M, device="cuda", weights=w)
            ref, out = _call_both(H, op, inp, M)
            for k in ("R2", "rrms", "inj_next", "x"):
                assert torch.equal(ref[k], out[k]), (kind, M, k)
        op.close()


def test_noalloc_size_limit(H):
    """A call whose plan needs more than the scratch holds is rejected before
    any launch (outputs untouched); M = 0 does nothing."""
    op = H.HCGR(H.Config(), 0)
    M = 16384
    assert H.hcgr_workspace_size(op.handle, M) > H.hcgr_noalloc_scratch_bytes()
    inp = synth.make_inputs(M, synth.Shape(), seed=1, device="cuda")
    out = op.alloc_outputs(M)
    out["x"].fill_(7.0)
    st = H.hcgr_forward_noalloc(op.handle, inp["R"], inp["y"], inp["inj"], inp["inj"].stride(0), inp["wnorm"],
                                inp["wd"], inp["wi"], inp["wu"], M, out["R2"], out["rrms"], out["inj_next"],
                                out["ld_inj_next"], out["x"], check=False)
    assert st == H.HCGR_ERR_WORKSPACE_TOO_SMALL
    assert "scratch" in H.last_error()
    torch.cuda.synchronize()
    assert bool((out["x"] == 7.0).all())
    assert H.hcgr_forward_noalloc(op.handle, None, None, None, 4, None, None, None, None, 0, None, None, None, 4,
                                  None) == H.HCGR_OK
    op.close()
