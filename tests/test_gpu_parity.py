"""GPU parity: the HIP path (called through the C ABI binding) against the
fp64 oracle on the same seeded inputs. Small and mid M are compared on every
row; the M=8192 and M=65536 workloads, in the configuration the benchmark
times, on sampled rows (every step is per token, so a row of a large call is
checked by running the oracle on that row alone)."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_all, check_r2, check_rrms, check_tol, to64

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


def run_oracle(inp, rows=None, merged=False, n_pad=0, wnorm_full=False, wd_key="wd"):
    cfg = oracle.OracleConfig(wnorm_full=wnorm_full, merged=merged, n_pad=n_pad)
    R, y, inj = inp["R"], inp["y"], inp["inj"]
    if rows is not None:
        idx = torch.as_tensor(rows, device=R.device)
        R, y, inj = R[idx], y[idx], inj[idx]
    return oracle.forward(cfg, R.cpu(), y.cpu(), inj.cpu().contiguous(), inp["wnorm"].cpu(), inp[wd_key].cpu(),
                          None if merged else inp["wi"].cpu(), inp["wu"].cpu(),
                          ld_inj=inj.shape[1])


def gpu_forward(op, inp, *, wd=None, wi="default", ld_next=None):
    M = inp["R"].shape[0]
    out = op.alloc_outputs(M, ld_next)
    op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"] if wd is None else wd,
               inp["wi"] if wi == "default" else wi, inp["wu"], out=out)
    torch.cuda.synchronize()
    return out


def sample_rows(M, n=96, seed=1):
    rng = np.random.default_rng(seed)
    rows = {0, 1, M // 2, M - 2, M - 1} | set(rng.choice(M, size=min(n, M), replace=False).tolist())
    return np.array(sorted(r for r in rows if 0 <= r < M))


SWEEP = [1, 2, 3, 4, 5, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 224, 257, 512, 1000,
         1024, 1025]


@pytest.mark.parametrize("M", SWEEP)
def test_token_sweep_every_row(op, weights, M):
    _say(f"[parity] sweep M={M} plan: {__import__('skinny_gemm_hcgr_amd').hcgr_describe_plan(op.cfg, M)}")
    inp = synth.make_inputs(M, SHAPE, seed=0, device="cuda", weights=weights)
    out = gpu_forward(op, inp)
    ref = run_oracle(inp)
    check_all(out, ref)


@pytest.mark.parametrize("M", [2048, 4095, 4096, 8192, 16384, 65536])
def test_token_sweep_sampled_rows(op, weights, M):
    _say(f"[parity] sampled M={M}")
    inp = synth.make_inputs(M, SHAPE, seed=0, device="cuda", weights=weights)
    out = gpu_forward(op, inp)
    rows = sample_rows(M)
    check_all(out, run_oracle(inp, rows), rows)


def test_beyond_4gib(op, weights):
    """R and R2 past 4 GiB (215000 tokens x 20480 bytes): every address the
    kernels form is 64-bit. Rows on both sides of the 4 GiB mark and the
    ragged last tile match the oracle, and the combine entry point gives the
    same R2 bit for bit."""
    M = 215000
    row_bytes = SHAPE.k * 2
    assert M * row_bytes > 1 << 32
    _say(f"[parity] beyond 4 GiB M={M}")
    inp = synth.make_inputs(M, SHAPE, seed=7, device="cuda", weights=weights)
    out = gpu_forward(op, inp)
    edge = (1 << 32) // row_bytes  # the row that straddles the 4 GiB mark
    rows = np.array(sorted(set(sample_rows(M, n=24).tolist()) | {edge - 1, edge, edge + 1, M - 1}))
    check_all(out, run_oracle(inp, rows), rows)
    R2 = op.combine(inp["R"], inp["y"], inp["inj"])
    torch.cuda.synchronize()
    idx = torch.as_tensor(rows, device="cuda")
    assert torch.equal(R2[idx], out["R2"][idx])


def test_decode_m1(op, weights):
    inp = synth.make_inputs(1, SHAPE, seed=0, device="cuda", weights=weights)
    check_all(gpu_forward(op, inp), run_oracle(inp))


def test_decode_m32(op, weights):
    inp = synth.make_inputs(32, SHAPE, seed=0, device="cuda", weights=weights)
    check_all(gpu_forward(op, inp), run_oracle(inp))


def tile_rows(M, tile=128, seed=3):
    """One row drawn from every `tile`-token tile of M (the last tile ragged),
    plus both ends of the first and last tiles."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, M, tile)
    ends = np.minimum(starts + tile, M)
    rows = {int(rng.integers(a, b)) for a, b in zip(starts, ends)} | {0, min(tile, M) - 1, int(starts[-1]), M - 1}
    return np.array(sorted(rows))


@pytest.mark.parametrize("M", [1, 7, 32, 100, 1024, 3000, 8192, 16384, 65536])
def test_merged_folded_n336(H, weights, M):
    """Merged 336-row down/inject weight with (1+Wnorm) folded in (the M=1024
    workload; also decode and large M, where the folded path has no other
    coverage). From 8192 tokens: one row of every 128-token tile."""
    _say(f"[parity] merged M={M}")
    o = H.HCGR(H.Config(weight_layout=H.HCGR_WEIGHTS_MERGED_FOLDED, n_pad=336), 0)
    inp = synth.make_inputs(M, SHAPE, seed=0, device="cuda", weights=weights)
    inp["wm"] = synth.fold_merged_weight(inp["wd"], inp["wi"], inp["wnorm"], 336, SHAPE.hs)
    out = gpu_forward(o, inp, wd=inp["wm"], wi=None)
    rows = None if M <= 1024 else sample_rows(M) if M < 8192 else tile_rows(M)
    check_all(out, run_oracle(inp, rows, merged=True, n_pad=336, wd_key="wm"), rows)
    o.close()


def test_prefill_m65536_every_tile(op, weights):
    """The M=65536 workload in the configuration the benchmark times: one row
    of every 128-token tile (the down kernel's tile-to-XCD grouping and the
    up kernel's channel ranges both index by tile) against the oracle."""
    M = 65536
    _say(f"[parity] every tile M={M}")
    inp = synth.make_inputs(M, SHAPE, seed=0, device="cuda", weights=weights)
    out = gpu_forward(op, inp)
    rows = tile_rows(M)
    assert len(rows) >= 512
    check_all(out, run_oracle(inp, rows), rows)


def test_prefill_m8192_stream0_x8(op, weights):
    """M=8192 with stream 0 of R scaled by 8 (per-stream RMS range), every row."""
    _say("[parity] M=8192 stream 0 x8, every row")
    inp = synth.make_inputs(8192, SHAPE, seed=0, device="cuda", weights=weights, scale_stream0=8.0)
    out = gpu_forward(op, inp)
    ref = run_oracle(inp)
    check_all(out, ref)
    r = to64(out["rrms"])
    assert np.all(r[:, 0] < r[:, 1:].min(axis=1))


def test_strided_injection_and_layer_chaining(op, weights):
    """inj_next written into a packed [M, 336] buffer (row stride 336) is fed
    back as the next call's inj, like consecutive layers; padding columns of
    the packed buffer must stay untouched."""
    M = 37
    inp = synth.make_inputs(M, SHAPE, seed=4, device="cuda", weights=weights, ld_inj=336)
    assert inp["inj"].stride(0) == 336
    out1 = gpu_forward(op, inp, ld_next=336)
    check_all(out1, run_oracle(inp))
    assert torch.all(out1["inj_next_buf"][:, 4:] == 0)
    y2 = synth.normal_bf16(9, 2, M, SHAPE.hs, device="cuda")
    inp2 = dict(inp, R=out1["R2"], y=y2, inj=out1["inj_next"])
    out2 = gpu_forward(op, inp2)
    check_all(out2, run_oracle(inp2))


@pytest.mark.parametrize("hs,r,M", [(1024, 512, 16384), (640, 64, 8192), (2560, 320, 16420), (640, 64, 260), (1024, 512, 1000)])
def test_tile_plan_shapes(H, hs, r, M):
    """Tile down kernel on other shapes: r = 512 (33 row blocks, two row
    splits per token tile), a short stream (HS = 640: 10 stages) with one
    stream per workgroup, a token count whose last tile is partial, and mid
    token counts whose streams are split into column segments (HS = 640: 5
    segments of 2 stages; r = 512: row splits and segments together)."""
    shape = synth.Shape(hs=hs, r=r)
    o = H.HCGR(H.Config(hs=hs, r=r), 0)
    plan = H.hcgr_describe_plan(o.cfg, M)
    _say(f"[parity] tile shapes hs={hs} r={r} M={M}: {plan}")
    assert "plan=tile" in plan
    inp = synth.make_inputs(M, shape, seed=11, device="cuda")
    out = gpu_forward(o, inp)
    rows = sample_rows(M, 64)
    cfg = oracle.OracleConfig(hs=hs, r=r)
    idx = torch.as_tensor(rows, device="cuda")
    ref = oracle.forward(cfg, inp["R"][idx].cpu(), inp["y"][idx].cpu(), inp["inj"][idx].cpu(), inp["wnorm"].cpu(),
                         inp["wd"].cpu(), inp["wi"].cpu(), inp["wu"].cpu())
    check_all(out, ref, rows)
    o.close()


@pytest.mark.parametrize("hs,r,M", [(256, 96, 4200), (512, 160, 4096), (384, 224, 4225), (256, 256, 4096),
                                    (512, 288, 5000), (2560, 320, 4096)])
def test_sweep_up_kernel_shapes(H, hs, r, M):
    """The up kernel that sweeps 32-channel groups with h held in registers,
    at every ring depth (2 to 5 k stages of 64), with half last stages
    (r % 64 == 32), one to five groups per channel range, uneven ranges and
    a last token tile of one token (M = 4225)."""
    shape = synth.Shape(hs=hs, r=r)
    o = H.HCGR(H.Config(hs=hs, r=r), 0)
    plan = H.hcgr_describe_plan(o.cfg, M)
    _say(f"[parity] sweep up kernel hs={hs} r={r} M={M}: {plan}")
    assert "k2_sweep" in plan
    inp = synth.make_inputs(M, shape, seed=13, device="cuda")
    out = gpu_forward(o, inp)
    rows = sample_rows(M, 64)
    cfg = oracle.OracleConfig(hs=hs, r=r)
    idx = torch.as_tensor(rows, device="cuda")
    ref = oracle.forward(cfg, inp["R"][idx].cpu(), inp["y"][idx].cpu(), inp["inj"][idx].cpu(), inp["wnorm"].cpu(),
                         inp["wd"].cpu(), inp["wi"].cpu(), inp["wu"].cpu())
    check_all(out, ref, rows)
    o.close()


@pytest.mark.parametrize("hs,r,M,kind", [(4352, 64, 1, "stream"), (4352, 64, 20, "stream"), (4224, 64, 8, "full"),
                                         (4224, 64, 64, "full")])
def test_fallback_plans_small_m(H, hs, r, M, kind):
    """Decode token counts whose stream width no decode K chunk divides (HS =
    34*128: 34 chunks of 128 are too many for the reduction, 512 does not
    divide it; HS = 33*128 likewise, with an odd stage count): the one-stream
    (partials summed by hcgr_k1_sum) and four-stream forms of hcgr_k1_full,
    then the staged up kernel."""
    shape = synth.Shape(hs=hs, r=r)
    o = H.HCGR(H.Config(hs=hs, r=r), 0)
    plan = H.hcgr_describe_plan(o.cfg, M)
    _say(f"[parity] fallback plan hs={hs} r={r} M={M}: {plan}")
    assert f"plan={kind}" in plan
    inp = synth.make_inputs(M, shape, seed=17, device="cuda")
    out = gpu_forward(o, inp)
    cfg = oracle.OracleConfig(hs=hs, r=r)
    ref = oracle.forward(cfg, inp["R"].cpu(), inp["y"].cpu(), inp["inj"].cpu(), inp["wnorm"].cpu(), inp["wd"].cpu(),
                         inp["wi"].cpu(), inp["wu"].cpu())
    check_all(out, ref)
    o.close()


GRID_SHAPES = [(128, 32), (384, 96), (640, 160), (1152, 224), (256, 512), (1408, 288)]
GRID_M = [1, 17, 65, 130, 700, 4100]


@pytest.mark.parametrize("hs,r,M", [(hs, r, M) for hs, r in GRID_SHAPES for M in GRID_M] +
                         [(128, 32, 16400), (640, 160, 16400)])
def test_shape_grid(H, hs, r, M):
    """Every plan and kernel variant across shapes: decode chunks that do or
    do not divide the stream (hs = 128 with M = 65 falls through to the tile
    plan), 1 to 11 column segments (some with a stage count that is not a
    multiple of four), row splits (r = 512), half last k stages in the up
    kernels (r % 64 == 32), both tiled up kernels, and four streams per down
    workgroup at M = 16400. Oracle on sampled rows."""
    shape = synth.Shape(hs=hs, r=r)
    o = H.HCGR(H.Config(hs=hs, r=r), 0)
    _say(f"[parity] grid hs={hs} r={r} M={M}: {H.hcgr_describe_plan(o.cfg, M)}")
    inp = synth.make_inputs(M, shape, seed=hs + r + M, device="cuda")
    out = gpu_forward(o, inp)
    rows = sample_rows(M, 24)
    cfg = oracle.OracleConfig(hs=hs, r=r)
    idx = torch.as_tensor(rows, device="cuda")
    ref = oracle.forward(cfg, inp["R"][idx].cpu(), inp["y"][idx].cpu(), inp["inj"][idx].cpu(), inp["wnorm"].cpu(),
                         inp["wd"].cpu(), inp["wi"].cpu(), inp["wu"].cpu())
    check_all(out, ref, rows)
    o.close()


@pytest.mark.parametrize("hs,r,M,kind", [(4096, 256, 1, "split"), (4096, 256, 32, "split"), (4096, 256, 100, "split"),
                                          (4096, 256, 145, "split"), (4096, 256, 146, "tile"), (1536, 192, 256, "split"),
                                          (7168, 512, 64, "split"), (7168, 512, 80, "tile")])
def test_split_limit_shapes(H, hs, r, M, kind):
    """The heuristic's shape-dependent plan choice: 3-row down blocks where
    they pad fewer 16-row blocks (r = 256, 512), and the split plan's token
    limit on both sides of it (145 tokens at HS = 4096, r = 256; 256 at
    HS = 1536; 64 at HS = 7168). Oracle on sampled rows."""
    shape = synth.Shape(hs=hs, r=r)
    o = H.HCGR(H.Config(hs=hs, r=r), 0)
    plan = H.hcgr_describe_plan(o.cfg, M)
    _say(f"[parity] split limit hs={hs} r={r} M={M}: {plan}")
    assert f"plan={kind}" in plan
    if kind == "split" and r in (256, 512):
        assert "row_blocks=3" in plan
    inp = synth.make_inputs(M, shape, seed=hs + r + M, device="cuda")
    out = gpu_forward(o, inp)
    rows = sample_rows(M, 24)
    cfg = oracle.OracleConfig(hs=hs, r=r)
    idx = torch.as_tensor(rows, device="cuda")
    ref = oracle.forward(cfg, inp["R"][idx].cpu(), inp["y"][idx].cpu(), inp["inj"][idx].cpu(), inp["wnorm"].cpu(),
                         inp["wd"].cpu(), inp["wi"].cpu(), inp["wu"].cpu())
    check_all(out, ref, rows)
    o.close()


def test_full_width_wnorm_large(H):
    """Wnorm indexed by k (length HC*HS) on the large-M path."""
    o = H.HCGR(H.Config(wnorm_len=SHAPE.k), 0)
    M = 16384
    inp = synth.make_inputs(M, SHAPE, seed=12, device="cuda", wnorm_full=True)
    out = gpu_forward(o, inp)
    rows = sample_rows(M, 48)
    check_all(out, run_oracle(inp, rows, wnorm_full=True), rows)
    o.close()


def test_full_width_wnorm(H):
    o = H.HCGR(H.Config(wnorm_len=SHAPE.k), 0)
    inp = synth.make_inputs(40, SHAPE, seed=5, device="cuda", wnorm_full=True)
    check_all(gpu_forward(o, inp), run_oracle(inp, wnorm_full=True))
    o.close()


@pytest.mark.parametrize("M", [3, 40, 300])
def test_wide_gates(op, M):
    """Unit-test variant with wider projections (Wd ~ N(0, 64/K), Wu ~ N(0, 4/r)) so
    that the gate spans (0, 1) and the up/sigmoid/mix path carries real weight."""
    inp = synth.make_inputs(M, SHAPE, seed=6, device="cuda", wd_std=8 / SHAPE.k ** 0.5, wu_std=2 / SHAPE.r ** 0.5)
    ref = oracle.forward(oracle.OracleConfig(), inp["R"].cpu(), inp["y"].cpu(), inp["inj"].cpu(), inp["wnorm"].cpu(),
                         inp["wd"].cpu(), inp["wi"].cpu(), inp["wu"].cpu(), debug=True)
    assert np.ptp(ref["G"]) > 0.9
    check_all(gpu_forward(op, inp), ref)


def test_r2_under_cancellation(op, weights):
    """R chosen as -bf16(y*iw) so that R2 = R + y*iw nearly cancels everywhere
    (|R2| <= 2^-8 |R|, down to ~1e-7 |R|): R2 must still be within one bf16 ulp of the
    exact value, which needs iw to better than fp32 precision."""
    M = 24
    inp = synth.make_inputs(M, SHAPE, seed=12, device="cuda", weights=weights)
    inj = inp["inj"].double().cpu()
    iw = 2.0 / (1.0 + torch.exp(-inj / SHAPE.hc))  # [M, HC]
    y = inp["y"].double().cpu()
    R = -(y[:, None, :] * iw[:, :, None]).reshape(M, SHAPE.k)
    inp["R"] = R.to(torch.bfloat16).cuda()
    out = gpu_forward(op, inp)
    ref = run_oracle(inp)
    ratio = np.abs(ref["R2"]) / np.abs(to64(inp["R"]))
    assert ratio.max() < 4e-3 and ratio.min() < 1e-6  # every element cancels to <= 2^-8 of |R|
    check_all(out, ref)


def test_zero_rows(op, weights):
    """All-zero rows: rrms = 1/sqrt(eps), x = 0, inj_next = 0."""
    inp = synth.make_inputs(20, SHAPE, seed=7, device="cuda", weights=weights)
    inp["R"][3:6] = 0
    inp["y"][3:6] = 0
    out = gpu_forward(op, inp)
    check_all(out, run_oracle(inp))
    assert torch.all(out["x"][3:6] == 0) and torch.all(out["inj_next"][3:6] == 0)


def test_deterministic(op, weights):
    for M in (5, 33, 2048):
        inp = synth.make_inputs(M, SHAPE, seed=8, device="cuda", weights=weights)
        a = gpu_forward(op, inp)
        b = gpu_forward(op, inp)
        for k in ("R2", "rrms", "inj_next", "x"):
            assert torch.equal(a[k], b[k]), (M, k)


def test_row_independence(op, weights):
    """A row of a large call equals the same row run alone: R2 bit for bit
    (same elementwise formula in every plan), the rest within tolerance."""
    inp = synth.make_inputs(1024, SHAPE, seed=9, device="cuda", weights=weights)
    big = gpu_forward(op, inp)
    for m in (0, 511, 1023):
        one = gpu_forward(op, dict(inp, R=inp["R"][m:m + 1], y=inp["y"][m:m + 1], inj=inp["inj"][m:m + 1]))
        assert torch.equal(one["R2"][0], big["R2"][m])
        check_rrms(one["rrms"][0], to64(big["rrms"][m]))
        check_tol(one["x"][0], to64(big["x"][m]), "x")
        check_tol(one["inj_next"][0], to64(big["inj_next"][m]), "inj_next")


def test_workspace_reuse_across_sizes(H, op, weights):
    """One workspace shared by calls of different M (different plans) in a row:
    a call's result does not depend on what an earlier call left behind."""
    ws = torch.empty(H.hcgr_workspace_size(op.handle, 2048) + 4096, dtype=torch.uint8, device="cuda")
    ws.fill_(0xFF)  # NaN patterns everywhere past the counters
    ws[:H.HCGR_WORKSPACE_COUNTER_BYTES].zero_()
    res = {}
    for M in (2048, 7, 300, 7, 33, 64, 16, 33):
        inp = synth.make_inputs(M, SHAPE, seed=10, device="cuda", weights=weights)
        out = op.alloc_outputs(M)
        op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], out=out,
                   workspace=ws)
        torch.cuda.synchronize()
        if M in res:
            for k in ("R2", "rrms", "inj_next", "x"):
                assert torch.equal(res[M][k], out[k]), (M, k)
        res[M] = out
    inp = synth.make_inputs(7, SHAPE, seed=10, device="cuda", weights=weights)
    check_all(res[7], run_oracle(inp))
    assert int(ws[:H.HCGR_WORKSPACE_COUNTER_BYTES].count_nonzero()) == 0  # every counter back at zero


def test_decode_interleaved_stress(H, op, weights):
    """Many back-to-back decode-size calls of four sizes interleaved on one
    workspace (cross-workgroup partials written by one kernel and summed by
    the next): bitwise-identical results every time, matching the oracle."""
    ws = H.new_workspace(H.hcgr_workspace_size(op.handle, 64))
    sizes = (5, 32, 64, 1)
    inps = {M: synth.make_inputs(M, SHAPE, seed=20 + M, device="cuda", weights=weights) for M in sizes}
    outs = {M: op.alloc_outputs(M) for M in sizes}
    first = {}
    for rep in range(25):
        for M in sizes:
            inp, out = inps[M], outs[M]
            op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], out=out,
                       workspace=ws)
            if rep == 0:
                torch.cuda.synchronize()
                first[M] = {k: out[k].clone() for k in ("R2", "rrms", "inj_next", "x")}
            elif rep % 6 == 0 or rep == 24:
                torch.cuda.synchronize()
                for k in first[M]:
                    assert torch.equal(first[M][k], out[k]), (rep, M, k)
    torch.cuda.synchronize()
    for M in sizes:
        check_all(outs[M], run_oracle(inps[M]))


@pytest.mark.parametrize("M", [32, 1024, 16384])
def test_forward_timed_matches_forward(H, op, weights, M):
    """The timed entry point gives the same bits as hcgr_forward and a start/end
    event pair per stage (an empty middle interval when the plan has no
    reduction kernel)."""
    inp = synth.make_inputs(M, SHAPE, seed=3, device="cuda", weights=weights)
    ref = gpu_forward(op, inp)
    out = op.alloc_outputs(M)
    ws = H.new_workspace(H.hcgr_workspace_size(op.handle, M))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for e in ev:
        e.record()
    torch.cuda.synchronize()
    H.hcgr_forward_timed(op.handle, inp["R"], inp["y"], inp["inj"], inp["inj"].stride(0), inp["wnorm"], inp["wd"],
                         inp["wi"], inp["wu"], M, out["R2"], out["rrms"], out["inj_next"], out["ld_inj_next"], out["x"],
                         ws, ws.numel(), torch.cuda.current_stream().cuda_stream, [e.cuda_event for e in ev])
    torch.cuda.synchronize()
    for k in ("R2", "rrms", "inj_next", "x"):
        assert torch.equal(ref[k], out[k]), k
    d = [ev[2 * i].elapsed_time(ev[2 * i + 1]) for i in range(3)]
    assert d[0] > 0 and d[2] > 0 and d[1] >= 0, d
    assert all(ev[2 * i + 1].elapsed_time(ev[2 * i + 2]) >= 0 for i in range(2))  # stages in order
    with pytest.raises(H.HcgrError):
        H.hcgr_forward_timed(op.handle, inp["R"], inp["y"], inp["inj"], inp["inj"].stride(0), inp["wnorm"], inp["wd"],
                             inp["wi"], inp["wu"], M, out["R2"], out["rrms"], out["inj_next"], out["ld_inj_next"],
                             out["x"], ws, ws.numel(), torch.cuda.current_stream().cuda_stream,
                             [e.cuda_event for e in ev[:5]] + [0])


@pytest.mark.parametrize("M", [48, 4160])
def test_graph_capture_replays(op, weights, M):
    """hcgr_forward captured into a HIP graph: several replays with new input
    values written between them, each checked against an eager call (bitwise)
    and the first against the oracle. M = 48 is the decode plan; M = 4160 the
    tile plan with column segments, the segment sum and the sweeping up
    kernel (oracle on sampled rows)."""
    inp = synth.make_inputs(M, SHAPE, seed=11, device="cuda", weights=weights)
    out = op.alloc_outputs(M)
    ws = op.workspace(M)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], out=out,
                   workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        op.forward(inp["R"], inp["y"], inp["inj"], inp["wnorm"], inp["wd"], inp["wi"], inp["wu"], out=out,
                   workspace=ws)
    for rep in range(4):
        fresh = synth.make_inputs(M, SHAPE, seed=100 + rep, device="cuda", weights=weights)
        inp["R"].copy_(fresh["R"])
        inp["y"].copy_(fresh["y"])
        inp["inj"].copy_(fresh["inj"])
        g.replay()
        torch.cuda.synchronize()
        eager = gpu_forward(op, fresh)
        for k in ("R2", "rrms", "inj_next", "x"):
            assert torch.equal(out[k], eager[k]), (rep, k)
        if rep == 0:
            if M <= 64:
                check_all(out, run_oracle(fresh))
            else:
                rows = sample_rows(M, 48)
                check_all(out, run_oracle(fresh, rows), rows)


def test_m0_and_errors_on_device(H, op, weights):
    z = torch.empty(0, SHAPE.k, dtype=torch.bfloat16, device="cuda")
    assert H.hcgr_forward(op.handle, z, None, None, 4, None, None, None, None, 0, None, None, None, 4, None,
                          None, 0) == H.HCGR_OK
    inp = synth.make_inputs(4, SHAPE, seed=0, device="cuda", weights=weights)
    out = op.alloc_outputs(4)
    ws = op.workspace(4)
    with pytest.raises(H.HcgrError) as e:  # R2 aliasing R
        H.hcgr_forward(op.handle, inp["R"], inp["y"], inp["inj"], 4, inp["wnorm"], inp["wd"], inp["wi"], inp["wu"],
                       4, inp["R"], out["rrms"], out["inj_next"], 4, out["x"], ws, ws.numel())
    assert e.value.status == H.HCGR_ERR_ALIASING
    out["x"].fill_(7.0)
    before = out["x"].clone()
    with pytest.raises(H.HcgrError) as e:  # workspace too small: nothing written
        H.hcgr_forward(op.handle, inp["R"], inp["y"], inp["inj"], 4, inp["wnorm"], inp["wd"], inp["wi"], inp["wu"],
                       4, out["R2"], out["rrms"], out["inj_next"], 4, out["x"], ws, 16)
    assert e.value.status == H.HCGR_ERR_WORKSPACE_TOO_SMALL
    torch.cuda.synchronize()
    assert torch.equal(before, out["x"])


@pytest.mark.parametrize("hs,r,M", [(8192, 320, 1), (8192, 320, 32), (8192, 320, 300), (40960, 320, 2),
                                    (40960, 320, 40), (40960, 64, 130)])
def test_wide_stream(H, hs, r, M):
    """Wide streams (HS = 8192 and 40960, the widths the pages' wide-stream
    test uses): at decode sizes the stream splits into more K chunks than the
    decode reduction takes, so the stream-wise fallback down kernels run; the
    tile plan above. Every row against the oracle."""
    shape = synth.Shape(hs=hs, r=r)
    o = H.HCGR(H.Config(hs=hs, r=r), 0)
    _say(f"[parity] wide stream hs={hs} r={r} M={M}: {H.hcgr_describe_plan(o.cfg, M)}")
    inp = synth.make_inputs(M, shape, seed=19, device="cuda")
    out = gpu_forward(o, inp)
    cfg = oracle.OracleConfig(hs=hs, r=r)
    ref = oracle.forward(cfg, inp["R"].cpu(), inp["y"].cpu(), inp["inj"].cpu(), inp["wnorm"].cpu(), inp["wd"].cpu(),
                         inp["wi"].cpu(), inp["wu"].cpu())
    check_all(out, ref)
    o.close()
