"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one.

Each mutant is an exact text substitution in ``oracle/hcgr_oracle.c`` (it must
match exactly once, so this test breaks loudly if the oracle is edited). The
mutated copy is compiled with gcc into a temporary directory and the whole
pin suite runs against it in a child process (so a crash in a mutant cannot
take pytest down); at least one pin must fail. Everything here runs on the
CPU; nothing touches the GPU library.
"""

from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hcgr_oracle.c")

# (name, exact text in the oracle, replacement)
MUTANTS = [
    ("iw_missing_factor_2", "iw[s] = 2.0 * logistic(widen_bf16(im[s]) / HC);",
     "iw[s] = logistic(widen_bf16(im[s]) / HC);"),
    ("iw_missing_div_hc", "iw[s] = 2.0 * logistic(widen_bf16(im[s]) / HC);",
     "iw[s] = 2.0 * logistic(widen_bf16(im[s]));"),
    ("sigmoid_sign", "return 1.0 / (1.0 + exp(-v));", "return 1.0 / (1.0 + exp(v));"),
    ("iw_wrong_stream", "widen_bf16(ym[c]) * iw[s];", "widen_bf16(ym[c]) * iw[HC - 1 - s];"),
    ("iw_by_channel", "widen_bf16(ym[c]) * iw[s];", "widen_bf16(ym[c]) * iw[c % HC];"),
    ("inj_stride_ignored", "const uint16_t* im = inj + m * ld_inj;",
     "const uint16_t* im = inj + m * HC;"),
    ("rms_eps_dropped", "rr[s] = 1.0 / sqrt(ms + cfg->eps);", "rr[s] = 1.0 / sqrt(ms);"),
    ("rms_sum_not_mean", "double ms = sq / HS;", "double ms = sq;"),
    ("rms_eps_outside_sqrt", "rr[s] = 1.0 / sqrt(ms + cfg->eps);",
     "rr[s] = 1.0 / (sqrt(ms) + cfg->eps);"),
    ("rms_no_sqrt", "rr[s] = 1.0 / sqrt(ms + cfg->eps);", "rr[s] = 1.0 / (ms + cfg->eps);"),
    ("rms_running_over_streams",
     "for (int s = 0; s < HC; ++s) {\n                double sq = 0.0;",
     "double sq = 0.0;\n            for (int s = 0; s < HC; ++s) {"),
    ("rrms_stream0_everywhere", "xn[k] = r2[k] * rr[s] * (1.0 + wn);",
     "xn[k] = r2[k] * rr[0] * (1.0 + wn);"),
    ("norm_missing_one_plus", "xn[k] = r2[k] * rr[s] * (1.0 + wn);", "xn[k] = r2[k] * rr[s] * wn;"),
    ("wnorm_full_by_channel", "double wn = cfg->wnorm_full ? Wn[k] : Wn[c];",
     "double wn = cfg->wnorm_full ? Wn[c] : Wn[c];"),
    ("down_uses_r2", "const double* act = cfg->merged ? u : xn;",
     "const double* act = cfg->merged ? u : r2;"),
    ("merged_refolds", "const double* act = cfg->merged ? u : xn;",
     "const double* act = cfg->merged ? xn : xn;"),
    ("down_transposed",
     "for (int64_t k = 0; k < K; ++k) acc += act[k] * wrow[k];\n                lora[j] = acc;",
     "for (int64_t k = 0; k < K; ++k) acc += act[k] * Wd[k * RR + j];\n                lora[j] = acc;"),
    ("merged_inject_row_offset", "(Wd + (int64_t)(RR + t) * K)", "(Wd + (int64_t)(RR + t + 1) * K)"),
    ("inject_scaled", "inj_next_out[m * HC + t] = acc;", "inj_next_out[m * HC + t] = acc / HC;"),
    ("silu_as_sigmoid", "h[j] = zj * logistic(zj);", "h[j] = logistic(zj);"),
    ("silu_missing_div_hc", "double zj = lora[j] / HC;", "double zj = lora[j];"),
    ("up_transposed", "for (int j = 0; j < RR; ++j) acc += h[j] * wrow[j];",
     "for (int j = 0; j < RR; ++j) acc += h[j] * Wu[(int64_t)j * K + k];"),
    ("gate_no_sigmoid", "G[k] = logistic(acc);", "G[k] = acc;"),
    ("mix_channel_major_gate", "acc += G[(int64_t)s * HS + c] * xn[(int64_t)s * HS + c];",
     "acc += G[(int64_t)c * HC + s] * xn[(int64_t)s * HS + c];"),
    ("mix_sums_r2", "acc += G[(int64_t)s * HS + c] * xn[(int64_t)s * HS + c];",
     "acc += G[(int64_t)s * HS + c] * r2[(int64_t)s * HS + c];"),
    ("mix_missing_div_hc", "x_out[m * HS + c] = acc / HC;", "x_out[m * HS + c] = acc;"),
    ("mix_entry_stream0_residual", "r2[k] = widen_bf16(Rm[k]);", "r2[k] = widen_bf16(Rm[k % HS]);"),
    ("mix_entry_doubles_residual", "r2[k] = widen_bf16(Rm[k]);", "r2[k] = 2.0 * widen_bf16(Rm[k]);"),
    ("combine_entry_drops_injection",
     "if (R2_out) memcpy(R2_out + m * K, r2, sizeof(double) * K);\n                continue;",
     "if (R2_out) for (int64_t k = 0; k < K; ++k) R2_out[m * K + k] = widen_bf16(Rm[k]);\n                continue;"),
]

_CHILD = r"""
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle_pins
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin({lib!r})
    except Exception as e:  # AssertionError or a numerical blow-up
        failed.append(pin.__name__)
print("FAILED_PINS", ",".join(failed))
"""


def _run_mutant(name, old, new, workdir):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutant {name}: pattern found {src.count(old)} times"
    path = os.path.join(workdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(workdir, f"lib_{name}.so")
    oracle.build(src=path, out=lib)
    code = _CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    env = dict(os.environ, OMP_NUM_THREADS="1")
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                       timeout=600)
    line = [ln for ln in p.stdout.splitlines() if ln.startswith("FAILED_PINS")]
    if p.returncode != 0 or not line:
        return name, f"crashed (rc={p.returncode})"  # a crash also counts as caught
    return name, line[0].split(" ", 1)[1] if " " in line[0] else ""


def test_unmutated_copy_passes_every_pin():
    with tempfile.TemporaryDirectory() as wd:
        _, failed = _run_mutant("identity", "return 1.0 / (1.0 + exp(-v));",
                                "return 1.0 / (1.0 + exp(-v));", wd)
    assert failed == "", failed


def test_every_mutant_is_caught():
    with tempfile.TemporaryDirectory() as wd:
        with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            results = list(ex.map(lambda t: _run_mutant(*t, wd), MUTANTS))
    uncaught = [n for n, failed in results if failed == ""]
    assert not uncaught, f"mutants no pin catches: {uncaught}"
    # keep the per-mutant catch list visible in -v output
    for n, failed in results:
        print(f"{n}: {failed}")
