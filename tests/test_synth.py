"""The seeded input generator: SplitMix64 + Box-Muller as defined in synth/."""
import math

import numpy as np
import pytest
import torch

import synth


def test_torch_words_match_pure_python_definition():
    rows = torch.tensor([0, 1, 7, 123456], dtype=torch.int64)
    w = synth.uniform_words(42, 5, rows, 6)
    for i, r in enumerate(rows.tolist()):
        tkey = synth.splitmix64_out_py(42, 5 + 1)
        rkey = synth.splitmix64_out_py(tkey, r + 1)
        want = [synth.splitmix64_out_py(rkey, j + 1) for j in range(6)]
        got = [v & ((1 << 64) - 1) for v in w[i].tolist()]
        assert got == want


def test_splitmix_is_the_published_stream():
    # successive outputs of one stream: state advances by the golden gamma,
    # output = mix(state); the first output of seed 0 is mix(gamma)
    z = synth.GAMMA
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & ((1 << 64) - 1)
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & ((1 << 64) - 1)
    z ^= z >> 31
    assert synth.splitmix64_out_py(0, 1) == z


def test_prefix_and_row_addressing():
    a = synth.normal_bf16(0, 1, 40, 64)
    b = synth.normal_bf16(0, 1, 7, 64, row0=20)
    assert torch.equal(a[20:27], b)
    c = synth.normal_bf16(0, 1, 40, 64, chunk_rows=3)
    assert torch.equal(a, c)


def test_distribution_moments():
    x = synth.normal_bf16(1, 2, 256, 4096, mean=0.0, std=0.5).float()
    assert abs(x.mean().item()) < 0.005
    assert abs(x.std().item() - 0.5) < 0.005
    # Gaussian tail: |z| > 3 sigma in ~0.27% of draws
    frac = (x.abs() > 1.5).float().mean().item()
    assert 0.0015 < frac < 0.0040


def test_tensors_are_independent_streams():
    a = synth.normal_bf16(0, 1, 4, 256).float().reshape(-1)
    b = synth.normal_bf16(0, 2, 4, 256).float().reshape(-1)
    corr = float(np.corrcoef(a.numpy(), b.numpy())[0, 1])
    assert abs(corr) < 0.1


def test_workload_inputs_shapes_and_scaling():
    sh = synth.Shape(4, 64, 16)
    d = synth.make_inputs(3, sh, scale_stream0=8.0, ld_inj=7)
    base = synth.make_inputs(3, sh)
    assert d["R"].shape == (3, 256) and d["y"].shape == (3, 64) and d["inj"].shape == (3, 7)
    assert torch.equal(d["R"][:, :64].float(), 8 * base["R"][:, :64].float())
    assert torch.equal(d["R"][:, 64:], base["R"][:, 64:])
    assert torch.equal(d["inj"][:, :4], base["inj"])
    assert d["wd"].float().std().item() == pytest.approx(1 / math.sqrt(256), rel=0.1)


def test_fold_merged_weight_layout():
    sh = synth.Shape(4, 8, 4)
    w = synth.make_weights(sh)
    wm = synth.fold_merged_weight(w["wd"], w["wi"], w["wnorm"], 16, 8)
    assert wm.shape == (16, 32)
    assert torch.all(wm[8:] == 0)
    one = (1 + w["wnorm"].float()).repeat(4)
    assert torch.equal(wm[:4], (w["wd"].float() * one).to(torch.bfloat16))
    assert torch.equal(wm[4:8], (w["wi"].float() * one).to(torch.bfloat16))
