"""Pins of the fp64 oracle to facts other than itself.

Each ``pin_*`` function runs the oracle library at ``lib`` on a special input
whose result is fixed by a closed form, an invariant of the method, or a
one-hot special case that reduces a step to a lookup; it raises
AssertionError when the oracle disagrees. The method is the Hyper-Connection
Gated Residual op of ROCm/aiter pull request #5913 ("Two-stage
Hyper-Connection Gated Residual kernel", section "Technical Details"); each
pin names the step(s) it fixes and the mistakes it is meant to catch. The
same functions run against deliberately broken copies of the oracle in
``test_oracle_mutants.py`` to show that every planted mistake trips at least
one of them.

The pages print no worked numeric example, so no pin quotes a value from them.
"""

from __future__ import annotations

import math
from decimal import Decimal, getcontext

import numpy as np
import torch
from scipy.special import expit

import oracle
import synth

TINY = oracle.OracleConfig(hc=4, hs=16, r=8, eps=1e-6)


def bf(a) -> np.ndarray:
    """float values -> bf16 bit patterns (round to nearest even); callers pass exact values."""
    t = torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def widen(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_inputs(cfg: oracle.OracleConfig, m: int, seed: int = 3, *, wd_std=None, wu_std=None):
    sh = synth.Shape(cfg.hc, cfg.hs, cfg.r, cfg.eps)
    d = synth.make_inputs(m, sh, seed=seed, wnorm_full=cfg.wnorm_full, wd_std=wd_std, wu_std=wu_std)
    return {k: (synth.bf16_bits(v) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def run(lib, cfg, d, *, debug=True, ld_inj=None):
    return oracle.forward(cfg, d["R"], d["y"], d["inj"], d["wnorm"], d["wd"], d.get("wi"), d["wu"],
                          ld_inj=ld_inj if ld_inj is not None else d.get("ld_inj"), debug=debug,
                          lib_path=lib)


def close(a, b, rel=1e-13, abs_=0.0):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    err = np.abs(a - b)
    lim = rel * np.maximum(np.abs(a), np.abs(b)) + abs_
    assert np.all(err <= lim), f"max err {err.max():.3e} (limit {lim.max():.3e})"


# ---------------------------------------------------------------- COMBINE --
def pin_combine_inj_zero(lib):
    """(COMBINE) inj = 0 gives iw = 2*sigmoid(0) = 1, so R2[s,c] = R[s,c] + y[c]
    exactly (a sum of two bf16 values is exact in fp64). Catches a missing
    factor 2, a y indexed by k instead of c, a dropped y term."""
    d = rand_inputs(TINY, 3)
    d["inj"] = np.zeros_like(d["inj"])
    o = run(lib, TINY, d)
    R = widen(d["R"]).reshape(3, TINY.hc, TINY.hs)
    y = widen(d["y"]).reshape(3, 1, TINY.hs)
    assert np.array_equal(o["R2"].reshape(3, TINY.hc, TINY.hs), R + y)


def pin_combine_y_zero(lib):
    """(COMBINE) y = 0 leaves the residual unchanged: R2 = R exactly."""
    d = rand_inputs(TINY, 2)
    d["y"] = np.zeros_like(d["y"])
    o = run(lib, TINY, d)
    assert np.array_equal(o["R2"], widen(d["R"]).reshape(2, -1))


def pin_combine_iw_closed_form(lib):
    """(COMBINE) R = 0, y = 1, inj = (HC, -HC, 2HC, 0) gives R2[s,:] = iw[s] =
    2*sigmoid(inj[s]/HC) = 2e/(e+1), 2/(e+1), 2e^2/(e^2+1), 1. Catches a missing
    1/HC, a missing factor 2, a sign error in the sigmoid."""
    cfg = TINY
    e = math.e
    want = [2 * e / (e + 1), 2 / (e + 1), 2 * e * e / (e * e + 1), 1.0]
    d = rand_inputs(cfg, 1)
    d["R"] = np.zeros_like(d["R"])
    d["y"] = bf(np.ones(cfg.hs))[None, :]
    d["inj"] = bf([[cfg.hc, -cfg.hc, 2 * cfg.hc, 0]])
    o = run(lib, cfg, d)
    got = o["R2"].reshape(cfg.hc, cfg.hs)
    for s in range(cfg.hc):
        close(got[s], np.full(cfg.hs, want[s]), rel=1e-15)
    close(want[0] + want[1], 2.0, rel=1e-15)  # iw(a) + iw(-a) = 2


def pin_inj_row_stride(lib):
    """(COMBINE) the injection logits may be a strided view (row stride > HC):
    padding columns must never be read. Same result as the packed layout."""
    d = rand_inputs(TINY, 3)
    o1 = run(lib, TINY, d)
    ld = TINY.hc + 3
    wide = bf(np.full((3, ld), 1000.0))
    wide[:, :TINY.hc] = d["inj"].reshape(3, TINY.hc)
    d2 = dict(d, inj=wide, ld_inj=ld)
    o2 = run(lib, TINY, d2, ld_inj=ld)
    for k in ("R2", "rrms", "inj_next", "x"):
        assert np.array_equal(o1[k], o2[k]), k


# ---------------------------------------------------------------------- N --
def pin_rrms_constant_streams(lib):
    """(N) a stream whose R2 is constant a has mean square a^2, so
    rrms = 1/sqrt(a^2 + eps). Catches sum-instead-of-mean, a missing sqrt or
    eps, a rrms taken over the wrong group of elements."""
    cfg = TINY
    a = [0.5, 2.0, -3.0, 1.25]
    d = rand_inputs(cfg, 1)
    d["y"] = np.zeros_like(d["y"])
    d["R"] = bf(np.repeat(np.array(a), cfg.hs))[None, :]
    o = run(lib, cfg, d)
    close(o["rrms"][0], [1.0 / math.sqrt(v * v + cfg.eps) for v in a], rel=1e-15)
    # xn = a * rrms * (1 + Wnorm[c])
    wn = widen(d["wnorm"])
    for s in range(cfg.hc):
        close(o["xn"][0].reshape(cfg.hc, cfg.hs)[s], a[s] / math.sqrt(a[s] ** 2 + cfg.eps) * (1 + wn),
              rel=1e-15)


def pin_zero_row(lib):
    """(N) an all-zero row has mean square 0, so rrms = 1/sqrt(eps) (1000 for
    eps = 1e-6) and everything downstream is zero, except G = sigmoid(0) = 1/2."""
    cfg = TINY
    d = rand_inputs(cfg, 1)
    d["R"] = np.zeros_like(d["R"])
    d["y"] = np.zeros_like(d["y"])
    o = run(lib, cfg, d)
    close(o["rrms"], np.full((1, cfg.hc), 1.0 / math.sqrt(cfg.eps)), rel=1e-15)
    for k in ("xn", "lora", "h", "gate", "x", "inj_next"):
        assert np.all(o[k] == 0.0), k
    assert np.all(o["G"] == 0.5)


def pin_xn_unit_rms(lib):
    """(N) with Wnorm = 0 every stream of xn has RMS sqrt(ms/(ms+eps)), i.e. 1
    to within eps/(2 ms), even when one stream is scaled by 8 (the per-stream
    range stress of the M=8192 workload). Catches one RMS over the whole row,
    or rrms applied to the wrong stream."""
    cfg = oracle.OracleConfig(hc=4, hs=64, r=8)
    d = rand_inputs(cfg, 3)
    R = widen(d["R"]).reshape(3, cfg.hc, cfg.hs)
    R[:, 0] *= 8.0
    d["R"] = bf(R.reshape(3, -1))
    d["wnorm"] = np.zeros_like(d["wnorm"])
    o = run(lib, cfg, d)
    xn = o["xn"].reshape(3, cfg.hc, cfg.hs)
    rms = np.sqrt(np.mean(xn * xn, axis=2))
    assert np.all(np.abs(rms - 1.0) < 1e-5), rms
    ratio = o["rrms"][:, 1:] / o["rrms"][:, :1]
    assert np.all(ratio > 4.0), ratio  # stream 0 is 8x larger, its rrms ~8x smaller


def pin_wnorm_factor(lib):
    """(N) xn carries the factor (1 + Wnorm): a constant Wnorm = w scales xn by
    exactly (1 + w); a full-width Wnorm[K] holding per-stream constants w_s
    scales stream s by (1 + w_s); a full-width Wnorm that repeats the per-channel
    one gives the per-channel result. Catches a missing '1 +', a Wnorm indexed
    by k when it has HS entries, or by c when it has K."""
    cfg = TINY
    d = rand_inputs(cfg, 2)
    d0 = dict(d, wnorm=np.zeros(cfg.hs, np.uint16))
    o0 = run(lib, cfg, d0)
    o1 = run(lib, cfg, dict(d, wnorm=bf(np.full(cfg.hs, 0.5))))
    close(o1["xn"], 1.5 * o0["xn"], rel=1e-15)
    cfg_f = oracle.OracleConfig(hc=cfg.hc, hs=cfg.hs, r=cfg.r, eps=cfg.eps, wnorm_full=True)
    ws = [0.5, -0.25, 1.0, 0.125]
    of = run(lib, cfg_f, dict(d, wnorm=bf(np.repeat(np.array(ws), cfg.hs))))
    for s in range(cfg.hc):
        close(of["xn"].reshape(2, cfg.hc, cfg.hs)[:, s], (1 + ws[s]) * o0["xn"].reshape(2, cfg.hc, cfg.hs)[:, s],
              rel=1e-15)
    oc = run(lib, cfg, d)
    ot = run(lib, cfg_f, dict(d, wnorm=np.tile(d["wnorm"], cfg.hc)))
    for k in ("R2", "rrms", "xn", "x", "inj_next"):
        assert np.array_equal(oc[k], ot[k]), k


# ------------------------------------------------------------ G1, INJ, G2 --
def _perm_rows(n_rows, k, seed):
    rng = np.random.default_rng(seed)
    return rng.choice(k, size=n_rows, replace=False)


def pin_down_onehot(lib):
    """(G1) Wd row j = e_{k_j} turns the down projection into a lookup:
    lora[j] = xn[k_j] exactly, and h[j] = SiLU(xn[k_j]/HC) = z*expit(z).
    Catches a transposed Wd, a missing or misplaced 1/HC, a wrong activation."""
    cfg = TINY
    d = rand_inputs(cfg, 2)
    kj = _perm_rows(cfg.r, cfg.k, 11)
    wd = np.zeros((cfg.r, cfg.k), np.float32)
    wd[np.arange(cfg.r), kj] = 1.0
    d["wd"] = bf(wd)
    o = run(lib, cfg, d)
    assert np.array_equal(o["lora"], o["xn"][:, kj])
    z = o["xn"][:, kj] / cfg.hc
    close(o["h"], z * expit(z), rel=1e-14)


def pin_inj_onehot(lib):
    """(INJ) Wi row t = e_{k_t}: inj_next[t] = xn[k_t] exactly (no 1/HC).
    Catches a transposed Wi or a 1/HC applied to the injection logits."""
    cfg = TINY
    d = rand_inputs(cfg, 2)
    kt = _perm_rows(cfg.hc, cfg.k, 12)
    wi = np.zeros((cfg.hc, cfg.k), np.float32)
    wi[np.arange(cfg.hc), kt] = 1.0
    d["wi"] = bf(wi)
    o = run(lib, cfg, d)
    assert np.array_equal(o["inj_next"], o["xn"][:, kt])


def pin_up_onehot(lib):
    """(G2) Wu row k = e_{j_k}: gate[k] = h[j_k] exactly and G = expit(gate).
    Catches a transposed Wu or a wrong gate activation. Wd is widened so that
    h spans a useful range."""
    cfg = TINY
    d = rand_inputs(cfg, 2, wd_std=1.0)
    rng = np.random.default_rng(13)
    jk = rng.integers(0, cfg.r, size=cfg.k)
    wu = np.zeros((cfg.k, cfg.r), np.float32)
    wu[np.arange(cfg.k), jk] = 1.0
    d["wu"] = bf(wu)
    o = run(lib, cfg, d)
    assert np.array_equal(o["gate"], o["h"][:, jk])
    close(o["G"], expit(o["h"][:, jk]), rel=1e-15)
    assert np.ptp(o["G"]) > 0.2


# -------------------------------------------------------------------- MIX --
def pin_mix_wd_zero(lib):
    """(MIX) Wd = 0 gives h = 0, gate = 0, G = 1/2 everywhere, so
    x[c] = (1/HC) * sum_s xn[s,c] / 2. Catches a missing 1/HC, a MIX that sums
    R2 instead of xn, or channels and streams swapped in the sum."""
    cfg = TINY
    d = rand_inputs(cfg, 3)
    d["wd"] = np.zeros_like(d["wd"])
    o = run(lib, cfg, d)
    assert np.all(o["G"] == 0.5)
    xn = o["xn"].reshape(3, cfg.hc, cfg.hs)
    close(o["x"], 0.5 * xn.mean(axis=1), rel=1e-14)


def pin_mix_stream_gates(lib):
    """(MIX) per-stream gates: Wd one-hot so that h[j] = SiLU(xn[k_j]/HC), and
    Wu rows of stream s one-hot at column s, so G[s,c] = expit(h[s]) for every c.
    Then x[c] = (1/HC) * sum_s expit(h[s]) * xn[s,c]. Catches a gate or xn
    indexed as c*HC + s (channel-major) instead of s*HS + c."""
    cfg = TINY
    d = rand_inputs(cfg, 2)
    kj = _perm_rows(cfg.r, cfg.k, 21)
    wd = np.zeros((cfg.r, cfg.k), np.float32)
    wd[np.arange(cfg.r), kj] = 4.0
    d["wd"] = bf(wd)
    wu = np.zeros((cfg.k, cfg.r), np.float32)
    for s in range(cfg.hc):
        wu[s * cfg.hs:(s + 1) * cfg.hs, s] = 1.0
    d["wu"] = bf(wu)
    o = run(lib, cfg, d)
    g = expit(o["h"][:, :cfg.hc])  # [M, HC]
    xn = o["xn"].reshape(2, cfg.hc, cfg.hs)
    want = (g[:, :, None] * xn).sum(axis=1) / cfg.hc
    close(o["x"], want, rel=1e-14)
    assert np.ptp(g) > 0.05


# ------------------------------------------------------------- invariants --
def pin_stream_permutation(lib):
    """All steps: permuting the streams (R blocks, inj entries, Wd/Wi column
    blocks, Wu row blocks, full-width Wnorm blocks) permutes R2 and rrms and
    leaves lora, h, inj_next and x unchanged. Catches any index that mixes up
    streams and channels on a non-symmetric input."""
    cfg = oracle.OracleConfig(hc=4, hs=16, r=8, wnorm_full=True)
    d = rand_inputs(cfg, 2, wd_std=0.5, wu_std=1.0)
    perm = np.array([2, 0, 3, 1])
    hs, hc, k = cfg.hs, cfg.hc, cfg.k

    def pk(a):  # permute stream blocks along the last (K) axis
        return a.reshape(*a.shape[:-1], hc, hs)[..., perm, :].reshape(*a.shape[:-1], k)

    dp = dict(d)
    dp["R"] = pk(d["R"])
    dp["inj"] = d["inj"].reshape(2, hc)[:, perm]
    dp["wd"] = pk(d["wd"])
    dp["wi"] = pk(d["wi"])
    dp["wnorm"] = pk(d["wnorm"])
    dp["wu"] = d["wu"].reshape(hc, hs, cfg.r)[perm].reshape(k, cfg.r)
    o = run(lib, cfg, d)
    op = run(lib, cfg, dp)
    close(op["R2"], pk(o["R2"]), rel=1e-15)
    close(op["rrms"], o["rrms"][:, perm], rel=1e-15)
    for key in ("lora", "h", "inj_next", "x"):
        close(op[key], o[key], rel=1e-12, abs_=1e-14)


def pin_scale_invariance(lib):
    """(N) with eps = 0, scaling R and y by 2 doubles R2 exactly, halves rrms,
    and leaves xn and everything after it unchanged. Catches rrms taken as
    1/ms or 1/sqrt(sum) and similar power mistakes."""
    cfg = oracle.OracleConfig(hc=4, hs=16, r=8, eps=0.0)
    d = rand_inputs(cfg, 2)
    d2 = dict(d, R=bf(2 * widen(d["R"])), y=bf(2 * widen(d["y"])))
    o = run(lib, cfg, d)
    o2 = run(lib, cfg, d2)
    assert np.array_equal(o2["R2"], 2 * o["R2"])
    close(o2["rrms"], 0.5 * o["rrms"], rel=1e-15)
    for key in ("xn", "lora", "h", "inj_next", "x"):
        close(o2[key], o[key], rel=1e-13, abs_=1e-15)


def pin_row_independence(lib):
    """Every step is per token: an M-row call equals M one-row calls, bit for bit."""
    cfg = TINY
    d = rand_inputs(cfg, 3)
    o = run(lib, cfg, d)
    for m in range(3):
        dm = dict(d, R=d["R"][m:m + 1], y=d["y"][m:m + 1], inj=d["inj"][m:m + 1])
        om = run(lib, cfg, dm)
        for k in ("R2", "rrms", "inj_next", "x"):
            assert np.array_equal(om[k][0], o[k][m]), (m, k)


# ---------------------------------------------------------- merged layout --
def _merge(d, cfg, n_pad, fold: bool):
    wd, wi, wn = (synth.from_bf16_bits(d[k]) for k in ("wd", "wi", "wnorm"))
    if fold:
        wm = synth.fold_merged_weight(wd, wi, wn, n_pad, cfg.hs)
    else:
        wm = torch.zeros((n_pad, cfg.k), dtype=torch.bfloat16)
        wm[:cfg.r] = wd
        wm[cfg.r:cfg.r + cfg.hc] = wi
    return synth.bf16_bits(wm)


def pin_merged_matches_separate(lib):
    """Merged layout (rows 0..r-1 Wd, r..r+HC-1 Wi, padding after; the caller
    folded (1 + Wnorm) into the columns): with Wnorm = 0 the fold is the
    identity and the merged call equals the separate one bit for bit. With a
    random Wnorm it matches to within the bf16 rounding of the fold. Catches a
    wrong inject-row offset, padding rows read, or (1 + Wnorm) applied twice."""
    cfg = oracle.OracleConfig(hc=4, hs=64, r=16)
    n_pad = 32
    cfg_m = oracle.OracleConfig(hc=4, hs=64, r=16, merged=True, n_pad=n_pad)
    d = rand_inputs(cfg, 3)
    d0 = dict(d, wnorm=np.zeros_like(d["wnorm"]))
    o = run(lib, cfg, d0)
    wm = _merge(d0, cfg, n_pad, fold=False)
    wm_pad = wm.copy()
    wm_pad[cfg.r + cfg.hc:] = bf(np.full((n_pad - cfg.r - cfg.hc, cfg.k), 7.0))
    om = run(lib, cfg_m, dict(d0, wd=wm_pad, wi=None))
    for k in ("R2", "rrms", "inj_next", "x", "lora", "h"):
        assert np.array_equal(o[k], om[k]), k
    # Wnorm = 1: the fold doubles every weight, which is exact in bf16 and fp64,
    # so the two layouts must again agree bit for bit.
    d1 = dict(d, wnorm=bf(np.ones(cfg.hs)))
    o = run(lib, cfg, d1)
    om = run(lib, cfg_m, dict(d1, wd=_merge(d1, cfg, n_pad, fold=True), wi=None))
    for k in ("R2", "rrms", "inj_next", "x", "lora", "h"):
        assert np.array_equal(o[k], om[k]), k
    o = run(lib, cfg, d)
    om = run(lib, cfg_m, dict(d, wd=_merge(d, cfg, n_pad, fold=True), wi=None))
    for k in ("R2", "rrms", "x"):
        close(om[k], o[k], rel=0.0, abs_=1e-2 * np.abs(o[k]).max())
    for k in ("inj_next", "lora"):
        close(om[k], o[k], rel=0.0, abs_=2e-2 * np.abs(o[k]).max())


# ------------------------------------------------------ high precision -----
def _decimal_forward(cfg, R, y, inj, wn, wd, wi, wu):
    """The six steps evaluated token by token in 40-digit decimal arithmetic."""
    getcontext().prec = 40
    D = lambda v: Decimal(float(v))  # noqa: E731  (bf16 -> float64 is exact)
    one, two = Decimal(1), Decimal(2)

    def sig(v):
        return one / (one + (-v).exp())

    HC, HS, r = cfg.hc, cfg.hs, cfg.r
    K = HC * HS
    res = {"R2": [], "rrms": [], "inj_next": [], "x": []}
    for m in range(R.shape[0]):
        iw = [two * sig(D(inj[m, s]) / HC) for s in range(HC)]
        R2 = [D(R[m, s * HS + c]) + D(y[m, c]) * iw[s] for s in range(HC) for c in range(HS)]
        rr = []
        for s in range(HC):
            ms = sum(R2[s * HS + c] ** 2 for c in range(HS)) / HS
            rr.append(one / (ms + D(cfg.eps)).sqrt())
        xn = [R2[s * HS + c] * rr[s] * (one + D(wn[c])) for s in range(HC) for c in range(HS)]
        lora = [sum(xn[k] * D(wd[j, k]) for k in range(K)) for j in range(r)]
        injn = [sum(xn[k] * D(wi[t, k]) for k in range(K)) for t in range(HC)]
        h = [(lo / HC) * sig(lo / HC) for lo in lora]
        G = [sig(sum(h[j] * D(wu[k, j]) for j in range(r))) for k in range(K)]
        x = [sum(G[s * HS + c] * xn[s * HS + c] for s in range(HC)) / HC for c in range(HS)]
        res["R2"].append([float(v) for v in R2])
        res["rrms"].append([float(v) for v in rr])
        res["inj_next"].append([float(v) for v in injn])
        res["x"].append([float(v) for v in x])
    return {k: np.array(v) for k, v in res.items()}


def pin_decimal_small(lib):
    """HC=2, HS=8, r=4: the fp64 oracle agrees with a 40-digit decimal
    evaluation of the same six steps to 1e-12 relative. Catches accumulation
    or conversion faults that the invariants above are blind to."""
    cfg = oracle.OracleConfig(hc=2, hs=8, r=4)
    d = rand_inputs(cfg, 2, wd_std=0.7, wu_std=1.5)
    o = run(lib, cfg, d)
    ref = _decimal_forward(cfg, widen(d["R"]), widen(d["y"]), widen(d["inj"]), widen(d["wnorm"]),
                           widen(d["wd"]), widen(d["wi"]), widen(d["wu"]))
    for k in ref:
        close(o[k], ref[k], rel=1e-12, abs_=1e-15)


def pin_decimal_eight_streams(lib):
    """HC=8, HS=8, r=4: the oracle against the 40-digit decimal evaluation with
    eight streams (the 1/HC scales inside iw, SiLU and the gated mean, and the
    per-stream RMS groups, at a stream count other than 2 and 4)."""
    cfg = oracle.OracleConfig(hc=8, hs=8, r=4)
    d = rand_inputs(cfg, 2, wd_std=0.7, wu_std=1.5)
    o = run(lib, cfg, d)
    ref = _decimal_forward(cfg, widen(d["R"]), widen(d["y"]), widen(d["inj"]), widen(d["wnorm"]),
                           widen(d["wd"]), widen(d["wi"]), widen(d["wu"]))
    for k in ref:
        close(o[k], ref[k], rel=1e-12, abs_=1e-15)


# ------------------------------------------- combine and mix entry points --
def pin_combine_entry_closed_form(lib):
    """(COMBINE entry point) with logits (HC, -HC, 2HC, 0) the injection weights
    have the closed forms 2e/(e+1), 2/(e+1), 2e^2/(e^2+1) and 1, so R2 = R +
    y*iw for random bf16 R and y; the logits sit in a strided view (row stride
    HC + 3, padding 1000) that must not be read. Catches an entry point that
    skips the injection, reads the wrong stream's logit or ignores the stride."""
    cfg = TINY
    e = math.e
    iw = np.array([2 * e / (e + 1), 2 / (e + 1), 2 * e * e / (e * e + 1), 1.0])
    d = rand_inputs(cfg, 3)
    ld = cfg.hc + 3
    inj = bf(np.full((3, ld), 1000.0))
    inj[:, :cfg.hc] = bf([[cfg.hc, -cfg.hc, 2 * cfg.hc, 0]] * 3)
    o = oracle.combine(cfg, d["R"], d["y"], inj, ld_inj=ld, lib_path=lib)
    R = widen(d["R"]).reshape(3, cfg.hc, cfg.hs)
    y = widen(d["y"]).reshape(3, 1, cfg.hs)
    # the two sides' iw may differ in the last bit; where R and y*iw cancel that
    # shows against the (small) result, so the bound adds a few ulps of |y*iw|
    close(o["R2"].reshape(3, cfg.hc, cfg.hs), R + y * iw[None, :, None], rel=1e-15,
          abs_=4e-16 * 2 * np.abs(y).max())


def pin_mix_entry_decimal(lib):
    """(mix entry point) HC=2, HS=8, r=4: rrms, inj_next and x of the mix entry
    agree to 1e-12 relative with the 40-digit decimal evaluation of the six
    steps with y = 0 (then R2 = R whatever the logits). Catches a mix entry
    that injects, rescales or mis-indexes the residual."""
    cfg = oracle.OracleConfig(hc=2, hs=8, r=4)
    d = rand_inputs(cfg, 2, wd_std=0.7, wu_std=1.5)
    o = oracle.mix(cfg, d["R"], d["wnorm"], d["wd"], d["wi"], d["wu"], lib_path=lib)
    zero_y = np.zeros(d["y"].shape)
    ref = _decimal_forward(cfg, widen(d["R"]), zero_y, widen(d["inj"]), widen(d["wnorm"]),
                           widen(d["wd"]), widen(d["wi"]), widen(d["wu"]))
    for k in ("rrms", "inj_next", "x"):
        close(o[k], ref[k], rel=1e-12, abs_=1e-15)


def pin_mix_entry_wd_zero(lib):
    """(mix entry point) Wd = 0 and Wi = 0 give h = 0, G = 1/2, inj_next = 0,
    so x[c] = (1/(2 HC)) sum_s xn[s,c]; with Wnorm = 0 and a constant stream s
    equal to a_s, xn[s,c] = a_s/sqrt(a_s^2 + eps). Catches a mix entry that
    drops the norm or the gate."""
    cfg = TINY
    d = rand_inputs(cfg, 1)
    a = np.array([0.5, -2.0, 3.0, 0.25])
    R = np.repeat(a, cfg.hs)[None, :]
    o = oracle.mix(cfg, bf(R), bf(np.zeros(cfg.hs)), np.zeros_like(d["wd"]), np.zeros_like(d["wi"]),
                   d["wu"], lib_path=lib)
    xn = a / np.sqrt(a * a + cfg.eps)
    assert np.all(o["inj_next"] == 0.0)
    close(o["rrms"][0], 1.0 / np.sqrt(a * a + cfg.eps), rel=1e-15)
    close(o["x"][0], np.full(cfg.hs, xn.sum() / (2 * cfg.hc)), rel=1e-14)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
