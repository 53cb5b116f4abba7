"""C ABI boundary on the CPU: the library loads, exports every function that
include/hcgr.h declares, and its host-side argument checks (the error
contract) behave as documented. No GPU and no kernel launch is involved:
hcgr_validate runs the same checks as hcgr_forward on plain addresses."""
import os
import re

import pytest

import skinny_gemm_hcgr_amd as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hcgr.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(H.LIB_PATH):
        from skinny_gemm_hcgr_amd import build
        build.build()
    return H.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:hcgr_status|void|const char\*)\s+(hcgr_\w+)\s*\(", text, re.M)))


def test_header_declares_the_api():
    names = declared_functions()
    for n in ("hcgr_create", "hcgr_destroy", "hcgr_workspace_size", "hcgr_forward", "hcgr_validate",
              "hcgr_status_string", "hcgr_last_error"):
        assert n in names


def test_binding_constants_match_the_header():
    """Every integer #define of include/hcgr.h that the binding also defines
    has the same value there (plan kinds, variant counts, status codes...)."""
    import re
    defs = dict(re.findall(r"^#define (HCGR_\w+)\s+\(?(-?\d+)\)?", open(HEADER).read(), re.M))
    shared = [k for k in defs if hasattr(H, k)]
    assert "HCGR_SPLIT_VARIANTS" in shared and "HCGR_PLAN_PERSISTENT" in shared
    for k in shared:
        assert getattr(H, k) == int(defs[k]), k


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert H.status_string(H.HCGR_OK) == "HCGR_OK"
    assert H.status_string(H.HCGR_ERR_ALIASING) == "HCGR_ERR_ALIASING"
    assert H.status_string(99) == "HCGR_ERR_UNKNOWN"


CFG = H.Config()
MCFG = H.Config(weight_layout=H.HCGR_WEIGHTS_MERGED_FOLDED, n_pad=336)


class Layout:
    """Disjoint, 256-byte aligned fake addresses for one call (never dereferenced)."""

    def __init__(self, cfg, M, ld_inj=None, ld_next=None):
        K, HS, HC, r = cfg.k, cfg.hs, cfg.hc, cfg.r
        self.ld_inj = ld_inj or HC
        self.ld_next = ld_next or HC
        sizes = {"R": M * K * 2, "y": M * HS * 2, "inj": M * self.ld_inj * 2, "wnorm": (cfg.wnorm_len or HS) * 2,
                 "wd": (cfg.n_pad if cfg.merged else r) * K * 2, "wi": HC * K * 2, "wu": K * r * 2,
                 "R2": M * K * 2, "rrms": M * HC * 4, "inj_next": M * self.ld_next * 2, "x": M * HS * 2}
        self.ws_bytes = H.hcgr_workspace_size_for(cfg, M)
        sizes["ws"] = self.ws_bytes
        a = 1 << 32
        self.addr = {}
        for k, n in sizes.items():
            self.addr[k] = a
            a += (n + 4096 + 255) // 256 * 256
        if cfg.merged:
            self.addr["wi"] = None
        self.cfg, self.M = cfg, M

    def call(self, **over):
        a = dict(self.addr)
        a.update({k: v for k, v in over.items() if k in a})
        M = over.get("M", self.M)
        return H.hcgr_validate(over.get("cfg", self.cfg), a["R"], a["y"], a["inj"], over.get("ld_inj", self.ld_inj),
                               a["wnorm"], a["wd"], a["wi"], a["wu"], M, a["R2"], a["rrms"], a["inj_next"],
                               over.get("ld_next", self.ld_next), a["x"], a["ws"],
                               over.get("ws_bytes", self.ws_bytes))


@pytest.mark.parametrize("M", [1, 3, 32, 100, 1024, 8192, 65536])
def test_valid_calls_pass(lib, M):
    assert Layout(CFG, M).call() == H.HCGR_OK
    assert Layout(MCFG, M).call() == H.HCGR_OK
    assert Layout(CFG, M, ld_inj=336, ld_next=336).call() == H.HCGR_OK


def test_m_zero_is_a_no_op_even_with_null_pointers(lib):
    assert H.hcgr_validate(CFG, None, None, None, 4, None, None, None, None, 0, None, None, None, 4, None,
                           None, 0) == H.HCGR_OK
    assert H.hcgr_workspace_size_for(CFG, 0) == 0


def test_negative_m(lib):
    assert Layout(CFG, 4).call(M=-1) == H.HCGR_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("name", ["R", "y", "inj", "wnorm", "wd", "wi", "wu", "R2", "rrms", "inj_next", "x", "ws"])
def test_null_pointer(lib, name):
    L = Layout(CFG, 8)
    assert L.call(**{name: 0}) == H.HCGR_ERR_INVALID_ARGUMENT
    assert "NULL" in H.last_error()


@pytest.mark.parametrize("name,off", [("R", 8), ("y", 2), ("wd", 4), ("wi", 8), ("wu", 2), ("R2", 8), ("x", 2),
                                      ("wnorm", 2), ("rrms", 2), ("inj", 1), ("inj_next", 1), ("ws", 8)])
def test_misaligned_pointer(lib, name, off):
    L = Layout(CFG, 8)
    assert L.call(**{name: L.addr[name] + off}) == H.HCGR_ERR_INVALID_ARGUMENT
    assert "aligned" in H.last_error()


def test_leading_dimensions(lib):
    L = Layout(CFG, 8)
    assert L.call(ld_inj=3) == H.HCGR_ERR_INVALID_ARGUMENT
    assert L.call(ld_next=2) == H.HCGR_ERR_INVALID_ARGUMENT


def test_workspace_too_small(lib):
    L = Layout(CFG, 64)
    assert L.call(ws_bytes=L.ws_bytes - 1) == H.HCGR_ERR_WORKSPACE_TOO_SMALL


def test_wi_with_merged_layout_is_rejected(lib):
    L = Layout(MCFG, 8)
    assert L.call(wi=L.addr["wu"] + (1 << 30)) == H.HCGR_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("out,other", [("R2", "R"), ("R2", "x"), ("x", "y"), ("rrms", "R2"), ("inj_next", "inj"),
                                       ("x", "wu"), ("ws", "R"), ("inj_next", "x"), ("R2", "wnorm")])
def test_aliasing(lib, out, other):
    L = Layout(CFG, 16)
    assert L.call(**{out: L.addr[other]}) == H.HCGR_ERR_ALIASING
    assert out.replace("ws", "workspace") in H.last_error()


def test_partial_overlap_is_aliasing(lib):
    L = Layout(CFG, 16)
    # x starting inside the tail of R2
    assert L.call(x=L.addr["R2"] + 16 * CFG.k * 2 - 256) == H.HCGR_ERR_ALIASING
    # strided inj_next sharing rows with the inj input of the same call
    assert L.call(inj_next=L.addr["inj"] + 16) == H.HCGR_ERR_ALIASING


@pytest.mark.parametrize("kw,st", [
    (dict(hc=3), H.HCGR_ERR_UNSUPPORTED), (dict(hc=16), H.HCGR_ERR_UNSUPPORTED),
    (dict(hs=2500), H.HCGR_ERR_UNSUPPORTED),
    (dict(r=100), H.HCGR_ERR_UNSUPPORTED), (dict(r=1024), H.HCGR_ERR_UNSUPPORTED),
    (dict(hc=0), H.HCGR_ERR_INVALID_ARGUMENT), (dict(eps=-1.0), H.HCGR_ERR_INVALID_ARGUMENT),
    (dict(eps=float("nan")), H.HCGR_ERR_INVALID_ARGUMENT), (dict(wnorm_len=7), H.HCGR_ERR_INVALID_ARGUMENT),
    (dict(weight_layout=5), H.HCGR_ERR_INVALID_ARGUMENT),
    (dict(weight_layout=H.HCGR_WEIGHTS_MERGED_FOLDED, n_pad=300), H.HCGR_ERR_INVALID_ARGUMENT),
])
def test_config_errors(lib, kw, st):
    cfg = H.Config(**kw)
    with pytest.raises(H.HcgrError) as e:
        H.hcgr_workspace_size_for(cfg, 4)
    assert e.value.status == st


@pytest.mark.parametrize("hc", [1, 2, 8])
def test_other_stream_counts(lib, hc):
    """HC = 1, 2 and 8 are accepted; their plan is the split plan at decode
    sizes (the reduction over HC streams, the HC-generic decode up kernel),
    then the tile plan (one stream per down workgroup, the stream sum, the
    HC-generic up kernel); one workspace sized for the largest M serves every
    smaller one."""
    cfg = H.Config(hc=hc)
    for M in (1, 5, 32, 33, 64, 65, 1000, 8192):
        assert Layout(cfg, M).call() == H.HCGR_OK
        L = Layout(cfg, M)
        assert _mix(L) == H.HCGR_OK and _combine(L) == H.HCGR_OK
        d = H.hcgr_describe_plan(cfg, M)
        if M <= (94 if hc == 8 else 256):  # the split limit: M x K x padded rows < 6.5e8
            assert "plan=split" in d and "k2_decg" in d, d
        else:
            assert "plan=tile" in d and "k1_sum" in d and "k2_gen" in d, d
    for hs, r in ((2560, 320), (256, 96), (1024, 512)):
        c = H.Config(hc=hc, hs=hs, r=r)
        prev = 0
        for M in range(1, 400):
            n = H.hcgr_workspace_size_for(c, M)
            assert n >= prev, (hc, hs, r, M)
            prev = n


def test_full_width_wnorm_and_other_shapes_accepted(lib):
    assert Layout(H.Config(wnorm_len=10240), 5).call() == H.HCGR_OK
    assert Layout(H.Config(hs=512, r=64), 5).call() == H.HCGR_OK
    assert Layout(H.Config(hs=8192, r=512), 3).call() == H.HCGR_OK


def test_plan_description_and_workspace_size(lib):
    prev = 0
    for M in (1, 16, 17, 32, 64, 65, 128, 129, 300, 1024, 1025, 2048, 4096, 8192, 16384, 65536):
        n = H.hcgr_workspace_size_for(CFG, M)
        assert n > 0 and n % 256 == 0
        assert n >= prev  # one workspace sized for the largest M serves every smaller call
        prev = n
        d = H.hcgr_describe_plan(CFG, M)
        assert d.startswith(f"M={M} plan=")
    assert H.hcgr_describe_plan(CFG, 0) == "M=0: no launch"


def test_workspace_size_monotone_every_m(lib):
    for cfg in (CFG, H.Config(hs=640, r=64), H.Config(hs=1024, r=512)):
        prev = 0
        for M in range(1, 1200):
            n = H.hcgr_workspace_size_for(cfg, M)
            assert n >= prev, (cfg, M)
            prev = n


def test_create_without_gfx950_fails_cleanly(lib):
    # on a host without a gfx950 device hcgr_create must return an error, not crash
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(H.HcgrError) as e:
        H.hcgr_create(CFG, 0)
    assert e.value.status in (H.HCGR_ERR_HIP, H.HCGR_ERR_INVALID_ARGUMENT, H.HCGR_ERR_UNSUPPORTED)


# ------------------------------------------------ combine and mix entries --
def _combine(L, **over):
    a = dict(L.addr)
    a.update({k: v for k, v in over.items() if k in a})
    return H.hcgr_validate_combine(over.get("cfg", L.cfg), a["R"], a["y"], a["inj"], over.get("ld_inj", L.ld_inj),
                                   over.get("M", L.M), a["R2"])


def _mix(L, **over):
    a = dict(L.addr)
    a.update({k: v for k, v in over.items() if k in a})
    return H.hcgr_validate_mix(over.get("cfg", L.cfg), a["R"], a["wnorm"], a["wd"], a["wi"], a["wu"],
                               over.get("M", L.M), a["rrms"], a["inj_next"], over.get("ld_next", L.ld_next),
                               a["x"], a["ws"], over.get("ws_bytes", L.ws_bytes))


@pytest.mark.parametrize("M", [1, 32, 8192, 65536])
def test_combine_and_mix_valid_calls(lib, M):
    L = Layout(CFG, M, ld_inj=336)
    assert _combine(L) == H.HCGR_OK
    assert _mix(L) == H.HCGR_OK
    assert _mix(Layout(MCFG, M)) == H.HCGR_OK


def test_combine_errors(lib):
    L = Layout(CFG, 8)
    assert _combine(L, M=0, R=0, y=0, inj=0, R2=0) == H.HCGR_OK
    assert _combine(L, M=-1) == H.HCGR_ERR_INVALID_ARGUMENT
    for name in ("R", "y", "inj", "R2"):
        assert _combine(L, **{name: 0}) == H.HCGR_ERR_INVALID_ARGUMENT, name
    assert _combine(L, R2=L.addr["R2"] + 8) == H.HCGR_ERR_INVALID_ARGUMENT
    assert _combine(L, ld_inj=3) == H.HCGR_ERR_INVALID_ARGUMENT
    for other in ("R", "y", "inj"):
        assert _combine(L, R2=L.addr[other]) == H.HCGR_ERR_ALIASING, other
        assert "R2" in H.last_error()
    assert _combine(L, cfg=H.Config(hc=3)) == H.HCGR_ERR_UNSUPPORTED


def test_mix_errors(lib):
    L = Layout(CFG, 16)
    assert _mix(L, M=0, R=0, wnorm=0, wd=0, wi=0, wu=0, rrms=0, inj_next=0, x=0, ws=0) == H.HCGR_OK
    for name in ("R", "wnorm", "wd", "wi", "wu", "rrms", "inj_next", "x", "ws"):
        assert _mix(L, **{name: 0}) == H.HCGR_ERR_INVALID_ARGUMENT, name
    assert _mix(L, ld_next=3) == H.HCGR_ERR_INVALID_ARGUMENT
    assert _mix(L, ws_bytes=L.ws_bytes - 1) == H.HCGR_ERR_WORKSPACE_TOO_SMALL
    for out, other in (("x", "R"), ("rrms", "wu"), ("inj_next", "x"), ("ws", "R"), ("x", "wd")):
        assert _mix(L, **{out: L.addr[other]}) == H.HCGR_ERR_ALIASING, (out, other)
    # the inputs mix does not take may share memory with its outputs freely
    assert _mix(L, x=L.addr["y"], rrms=L.addr["R2"]) == H.HCGR_OK


def test_wait_polls_needs_a_handle(lib):
    """hcgr_set_wait_polls is pure host code: a NULL handle is rejected with
    the documented status and message."""
    with pytest.raises(H.HcgrError) as e:
        H.hcgr_set_wait_polls(None, 5)
    assert e.value.status == H.HCGR_ERR_INVALID_ARGUMENT
    assert "NULL" in H.last_error()
    assert H.HCGR_DEFAULT_WAIT_POLLS == 1 << 20 and H.HCGR_MAX_WAIT_POLLS == 1 << 24
