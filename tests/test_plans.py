"""Tuned plan tables on the CPU (pure host functions of the C ABI): the
candidate list, the lookup rule (nearest key in log space, the heuristic
below the smallest key and for heuristic entries, the heuristic wherever a
choice cannot run), rejection of malformed tables, and the table-aware
workspace bound."""
import os
import re

import pytest

import skinny_gemm_hcgr_amd as H

CFG = H.Config()


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(H.LIB_PATH):
        from skinny_gemm_hcgr_amd import build
        build.build()
    return H.load_library()


def tile(M, spw=1, seg=1, up=0, ranges=1):
    return {"tokens": M, "kind": H.HCGR_PLAN_TILE, "down_variant": 0, "streams_per_wg": spw, "segments": seg,
            "up_variant": up, "ranges": ranges}


def split(M, v):
    return {"tokens": M, "kind": H.HCGR_PLAN_SPLIT, "down_variant": v, "streams_per_wg": 0, "segments": 0,
            "up_variant": 0, "ranges": 0}


def ws_of(desc):
    return int(re.search(r"workspace=(\d+)", desc).group(1))


@pytest.mark.parametrize("cfg", [CFG, H.Config(hs=640, r=64), H.Config(hc=2, hs=1024, r=512),
                                 H.Config(weight_layout=H.HCGR_WEIGHTS_MERGED_FOLDED, n_pad=336)])
@pytest.mark.parametrize("M", [1, 32, 128, 129, 300, 4096, 65536])
def test_every_candidate_is_a_valid_one_entry_table(lib, cfg, M):
    cands = H.hcgr_plan_candidates(cfg, M)
    assert cands, (cfg, M)
    kinds = {c["kind"] for c in cands}
    assert H.HCGR_PLAN_TILE in kinds
    assert (H.HCGR_PLAN_SPLIT in kinds) == (M <= 256)
    for c in cands:
        assert c["tokens"] == M
        chosen, desc = H.hcgr_plan_lookup(cfg, [c], M)
        assert chosen == c, (chosen, c)
        assert desc.startswith(f"M={M} plan=")
        assert H.hcgr_workspace_size_table(cfg, [c], M) >= ws_of(desc)


def test_lookup_rule(lib):
    t = [tile(64, seg=4), {"tokens": 256, "kind": H.HCGR_PLAN_HEURISTIC}, tile(4096, spw=4, up=1, ranges=2)]
    expect = {1: 0, 63: 0, 64: 64, 100: 64, 128: 64, 129: 256, 1024: 256, 1025: 4096, 70000: 4096}
    for M, key in expect.items():
        chosen, desc = H.hcgr_plan_lookup(CFG, t, M)
        assert chosen["tokens"] == key, (M, chosen)
        if key in (0, 256):  # below the smallest key, or a heuristic entry
            assert chosen["kind"] == H.HCGR_PLAN_HEURISTIC
            assert desc == H.hcgr_describe_plan(CFG, M)
    assert "segments=4" in H.hcgr_plan_lookup(CFG, t, 100)[1]
    assert "streams/wg=4" in H.hcgr_plan_lookup(CFG, t, 70000)[1]
    assert H.hcgr_plan_lookup(CFG, [], 32)[1] == H.hcgr_describe_plan(CFG, 32)


def test_choice_that_cannot_run_falls_back(lib):
    # a decode-plan choice serves at most 256 tokens: above that the heuristic applies
    t = [split(128, 4)]
    assert H.hcgr_plan_lookup(CFG, t, 200)[0]["kind"] == H.HCGR_PLAN_SPLIT
    chosen, desc = H.hcgr_plan_lookup(CFG, t, 1000)
    assert chosen["kind"] == H.HCGR_PLAN_HEURISTIC and desc == H.hcgr_describe_plan(CFG, 1000)


@pytest.mark.parametrize("table", [
    [tile(64), tile(64)],                                  # keys not strictly increasing
    [tile(256), tile(64)],
    [tile(0)],                                             # key < 1
    [dict(tile(64), kind=7)],                              # unknown kind
    [split(512, 0)],                                       # decode plan above 256 tokens
    [split(32, H.HCGR_SPLIT_VARIANTS)],                     # no such down variant
    [tile(64, seg=3)],                                     # 3 does not divide HS/128 = 20
    [tile(64, spw=4, seg=2)],                              # segments with four streams per workgroup
    [tile(64, spw=2)],
    [tile(64, up=2)],                                      # stream-generic up kernel at HC = 4
    [tile(4096, up=1, ranges=0)], [tile(4096, up=1, ranges=81)],
    [tile(64, up=0, ranges=2)],                            # ranges without the sweep
])
def test_malformed_tables_are_rejected(lib, table):
    with pytest.raises(H.HcgrError) as e:
        H.hcgr_plan_lookup(CFG, table, 100)
    assert e.value.status == H.HCGR_ERR_INVALID_ARGUMENT
    with pytest.raises(H.HcgrError):
        H.hcgr_workspace_size_table(CFG, table, 100)


def test_other_stream_counts_reject_four_stream_choices(lib):
    c2 = H.Config(hc=2)
    assert H.hcgr_plan_lookup(c2, [split(16, 0)], 16)[0]["kind"] == H.HCGR_PLAN_SPLIT
    for bad in ([tile(64, spw=4)], [tile(64, up=0)]):
        with pytest.raises(H.HcgrError):
            H.hcgr_plan_lookup(c2, bad, 64)
    assert H.hcgr_plan_lookup(c2, [tile(64, seg=5, up=2)], 64)[0]["segments"] == 5


def test_workspace_bound_with_table(lib):
    """The table-aware bound covers the plan of every M' <= M and never
    decreases, whatever the table."""
    tables = [
        [tile(16, seg=20), split(100, 9), tile(300, seg=2), tile(2048, spw=4, up=1, ranges=8)],
        [split(1, 1), {"tokens": 64, "kind": H.HCGR_PLAN_HEURISTIC}, tile(5000, seg=20)],
        [tile(8192, seg=20, up=1, ranges=4)],
    ]
    for t in tables:
        prev = 0
        for M in list(range(1, 700, 7)) + [1000, 2047, 2048, 3000, 5000, 8191, 8192, 12000, 20000]:
            n = H.hcgr_workspace_size_table(CFG, t, M)
            need = ws_of(H.hcgr_plan_lookup(CFG, t, M)[1])
            assert n >= need, (t, M, n, need)
            assert n >= prev, (t, M)
            prev = n


def test_shipped_tables_load_and_validate(lib):
    """The tables shipped with the package (written by the tuner on an MI355X)
    match their configuration and pass the library's table checks: HC = 4
    with separate and merged/folded weights, HC = 1, 2, 8 with separate ones."""
    cfgs = [CFG, H.Config(weight_layout=H.HCGR_WEIGHTS_MERGED_FOLDED, n_pad=336)] + [H.Config(hc=hc) for hc in (1, 2, 8)]
    for cfg in cfgs:
        path = H.shipped_plan_table(cfg)
        assert path is not None, cfg
        t = H.load_plan_table(path, cfg)
        assert t and all(t[i]["tokens"] < t[i + 1]["tokens"] for i in range(len(t) - 1))
        for M in (1, 32, 100, 1000, 65536):
            H.hcgr_plan_lookup(cfg, t, M)
            assert H.hcgr_workspace_size_table(cfg, t, M) >= ws_of(H.hcgr_plan_lookup(cfg, t, M)[1])
    assert H.shipped_plan_table(H.Config(hs=1024)) is None


@pytest.mark.parametrize("hc", [1, 2, 4, 8])
@pytest.mark.parametrize("hs,r", [(2560, 320), (1024, 64), (4096, 512), (640, 96)])
def test_workspace_bound_covers_every_smaller_plan(lib, hc, hs, r):
    """hcgr_workspace_size_for(M) never decreases and is at least the need of
    the plan of every M' <= M, so a workspace sized for the largest M serves
    every smaller call (at HC = 1 the 64-token tile plan runs past 16384
    tokens, with more column segments at some counts than at larger ones)."""
    cfg = H.Config(hc=hc, hs=hs, r=r)
    Ms = sorted(set(list(range(1, 300)) + list(range(300, 40000, 61)) + [16383, 16384, 16448, 24576, 24577, 32640,
                                                                           32641, 40000, 65536]))
    prev, need_max = 0, 0
    for M in Ms:
        n = H.hcgr_workspace_size_for(cfg, M)
        need_max = max(need_max, ws_of(H.hcgr_describe_plan(cfg, M)))
        assert n >= prev, (M, n, prev)
        assert n >= need_max, (M, n, need_max)
        prev = n


def test_workspace_keeps_the_counter_bytes(lib):
    """Every plan's data starts past the counter bytes; the fused and
    persistent decode plans are tuned-table choices at every stream count."""
    for hc in (1, 2, 4, 8):
        cfg = H.Config(hc=hc)
        for M in (1, 16, 17, 32, 33, 100, 5000):
            d = H.hcgr_describe_plan(cfg, M)
            assert "plan=fused" not in d, d
            assert ws_of(d) > H.HCGR_WORKSPACE_COUNTER_BYTES
            for kind in (H.HCGR_PLAN_FUSED, H.HCGR_PLAN_PERSISTENT):
                if M <= 256:
                    c = {"tokens": M, "kind": kind, "down_variant": int(M > 16)}
                    chosen, desc = H.hcgr_plan_lookup(cfg, [c], M)
                    assert chosen["kind"] == kind, (hc, M, desc)
                    assert H.hcgr_workspace_size_table(cfg, [c], M) >= ws_of(desc)


# (M, down variant, HS, r) -> up-kernel channels and grid of the HC = 4 split
# plan: 10 channels where HS is a multiple of 2560 unless they need more
# rounds of workgroups than 16 (a round: the workgroups that fit the 256 CUs'
# LDS at once; 64-token tiles fit two per CU with 10 channels, one with 16;
# 32-token tiles two either way; 16-token tiles three and two)
@pytest.mark.parametrize("M,kd,hs,r,cw,tiles", [
    (1, 0, 2560, 320, 10, 1), (48, 0, 2560, 320, 10, 3),              # 16-token tiles: one round either way
    (64, 4, 2560, 320, 10, 2), (96, 4, 2560, 320, 16, 3),             # 32-token tiles: 768 of 10 need two rounds
    (128, 4, 2560, 320, 10, 4), (160, 4, 2560, 320, 16, 5),           # four tiles: two rounds either way
    (128, 8, 2560, 320, 10, 2), (192, 8, 2560, 320, 10, 3), (256, 8, 2560, 320, 10, 4),  # 64-token tiles
    (9, 1, 5120, 320, 10, 1), (30, 4, 1280, 320, 16, 1), (128, 8, 2560, 512, 10, 2),
])
def test_up_kernel_channel_rule(lib, M, kd, hs, r, cw, tiles):
    cfg = H.Config(hs=hs, r=r)
    table = [{"tokens": M, "kind": H.HCGR_PLAN_SPLIT, "down_variant": kd, "streams_per_wg": 0, "segments": 0,
              "up_variant": 0, "ranges": 0}]
    desc = H.hcgr_plan_lookup(cfg, table, M)[1]
    tm = (16, 16, 16, 16, 32, 32, 32, 32, 64, 64)[kd]
    assert f"k2_dec tm={tm} waves={(cw + 3) // 4} channels={cw} grid={hs // cw}x{tiles}" in desc, desc
