"""Seeded synthetic inputs for the Hyper-Connection Gated Residual (HCGR) op.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark. It holds none of the op's arithmetic: it only draws numbers and
rounds them to bf16. (The one exception-looking helper, ``fold_merged_weight``,
builds an *input* that a caller prepares before calling the op: the merged
down/inject matrix with the norm weight pre-multiplied into its columns, the
form the HCGR pull request (ROCm/aiter #5913, "Performance" section) says it
benchmarks with. Both sides consume that matrix as given; neither computes it.)

Generator (counter based, so any element can be drawn on its own and a smaller
M is always a prefix of a larger one):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014): the n-th output (n >= 1) of a stream seeded with
  ``s`` is ``mix(s + n*G)`` with ``G = 0x9E3779B97F4A7C15`` and ``mix`` the
  xor-shift-multiply finaliser with constants 0xBF58476D1CE4E5B9 and
  0x94D049BB133111EB (shifts 30, 27, 31), all modulo 2**64.
* keys: ``tkey = out_{tensor_id+1}(seed)``, ``rkey = out_{row+1}(tkey)``;
  element ``i`` of a row draws the 64-bit word ``out_{i+1}(rkey)``.
* uniform: ``u = ((w >> 11) + 0.5) * 2**-53`` in (0, 1).
* Box-Muller (1958) on element pairs ``(2p, 2p+1)``:
  ``z0 = sqrt(-2 ln u0) cos(2 pi u1)``, ``z1 = sqrt(-2 ln u0) sin(2 pi u1)``.
* value = ``mean + std * z`` in fp64, rounded to fp32 then to bf16, both
  round-to-nearest-even.

The implementation uses torch int64 tensors with explicit masking for the
logical shifts, so it runs unchanged on the CPU or on a GPU; every test feeds
the *same* generated tensor to both the oracle and the GPU path, so the two
devices never need to agree bit for bit (they are checked against a pure
Python rendering of the same definition in the test-suite anyway).
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch

__all__ = [
    "GAMMA",
    "splitmix64_out_py",
    "uniform_words",
    "normal_bf16",
    "TENSOR_IDS",
    "Shape",
    "WORKLOADS",
    "make_inputs",
    "fold_merged_weight",
    "bf16_bits",
    "from_bf16_bits",
]

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
_MIX1 = 0xBF58476D1CE4E5B9
_MIX2 = 0x94D049BB133111EB


def _signed(v: int) -> int:
    v &= MASK64
    return v - (1 << 64) if v >= (1 << 63) else v


def _mix_py(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * _MIX1) & MASK64
    z = ((z ^ (z >> 27)) * _MIX2) & MASK64
    return z ^ (z >> 31)


def splitmix64_out_py(seed: int, n: int) -> int:
    """n-th (n >= 1) SplitMix64 output of a stream seeded with ``seed`` (pure Python)."""
    return _mix_py((seed + n * GAMMA) & MASK64)


def _lsr(z: torch.Tensor, k: int) -> torch.Tensor:
    # logical right shift of an int64 tensor holding a uint64 bit pattern
    return (z >> k) & ((1 << (64 - k)) - 1)


def _mix_t(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _signed(_MIX1)
    z = (z ^ _lsr(z, 27)) * _signed(_MIX2)
    return z ^ _lsr(z, 31)


def uniform_words(seed: int, tensor_id: int, rows: torch.Tensor, ncols: int) -> torch.Tensor:
    """uint64 words (as int64 bit patterns) for elements ``[rows, 0:ncols]``."""
    tkey = splitmix64_out_py(seed, tensor_id + 1)
    r = rows.to(torch.int64).reshape(-1, 1)
    rkey = _mix_t(r * _signed(GAMMA) + _signed(tkey + GAMMA))  # out_{row+1}(tkey)
    i = torch.arange(ncols, dtype=torch.int64, device=rows.device).reshape(1, -1)
    return _mix_t(rkey + (i + 1) * _signed(GAMMA))


def _normal_rows(seed: int, tensor_id: int, rows: torch.Tensor, ncols: int) -> torch.Tensor:
    nc = ncols + (ncols & 1)
    w = uniform_words(seed, tensor_id, rows, nc)
    u = (_lsr(w, 11).to(torch.float64) + 0.5) * (2.0 ** -53)
    u0 = u[:, 0::2]
    u1 = u[:, 1::2]
    rho = torch.sqrt(-2.0 * torch.log(u0))
    th = (2.0 * math.pi) * u1
    z = torch.stack((rho * torch.cos(th), rho * torch.sin(th)), dim=-1).reshape(rows.numel(), nc)
    return z[:, :ncols]


def normal_bf16(seed: int, tensor_id: int, nrows: int, ncols: int, mean: float = 0.0,
                std: float = 1.0, device="cpu", row0: int = 0, chunk_rows: int = 2048) -> torch.Tensor:
    """bf16 tensor [nrows, ncols] of N(mean, std^2) draws; rows ``row0 .. row0+nrows-1``."""
    out = torch.empty((nrows, ncols), dtype=torch.bfloat16, device=device)
    step = max(1, min(chunk_rows, (1 << 24) // max(ncols, 1)))
    for a in range(0, nrows, step):
        b = min(nrows, a + step)
        rows = torch.arange(row0 + a, row0 + b, dtype=torch.int64, device=device)
        z = _normal_rows(seed, tensor_id, rows, ncols)
        out[a:b] = (mean + std * z).to(torch.float32).to(torch.bfloat16)
    return out


def bf16_bits(t: torch.Tensor):
    """numpy uint16 view of a bf16 tensor (copied to the CPU)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")


def from_bf16_bits(a) -> torch.Tensor:
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


# Tensor identifiers: part of the generator's definition (they select the stream).
TENSOR_IDS = {"R": 1, "y": 2, "inj": 3, "wnorm": 4, "wd": 5, "wi": 6, "wu": 7}


@dataclass(frozen=True)
class Shape:
    hc: int = 4
    hs: int = 2560
    r: int = 320
    eps: float = 1e-6

    @property
    def k(self) -> int:
        return self.hc * self.hs


@dataclass(frozen=True)
class Workload:
    name: str
    m: int
    merged: bool = False
    n_pad: int = 0
    scale_stream0: float = 1.0


# The five workloads of the HCGR study: decode M=1 and M=32, M=1024 with the
# merged/folded 336-row down+inject weight, M=8192 prefill with stream 0 of R
# scaled by 8, and the M=65536 long prefill.
WORKLOADS = {
    "decode_m1": Workload("decode_m1", 1),
    "decode_m32": Workload("decode_m32", 32),
    "merged_m1024": Workload("merged_m1024", 1024, merged=True, n_pad=336),
    "prefill_m8192_s0x8": Workload("prefill_m8192_s0x8", 8192, scale_stream0=8.0),
    "prefill_m65536": Workload("prefill_m65536", 65536),
}


def make_inputs(m: int, shape: Shape = Shape(), *, seed: int = 0, device="cpu",
                wnorm_full: bool = False, scale_stream0: float = 1.0,
                wd_std: float | None = None, wu_std: float | None = None,
                ld_inj: int | None = None, weights: dict | None = None) -> dict:
    """Seeded inputs for one call: R [m,K], y [m,HS], inj [m,ld_inj] (first HC
    columns meaningful), wnorm [HS] or [K], wd [r,K], wi [HC,K], wu [K,r].

    Distributions: R, y, inj ~ N(0,1); wnorm ~ N(0, 0.1^2); wd, wi ~ N(0, 1/K)
    (standard deviation 1/sqrt(K)); wu ~ N(0, 1/r). ``wd_std``/``wu_std`` widen the
    projections for tests that need the gate to span (0, 1). ``weights`` reuses
    previously drawn weight tensors (they do not depend on m).
    """
    hc, hs, r, k = shape.hc, shape.hs, shape.r, shape.k
    ld = hc if ld_inj is None else ld_inj
    out = {}
    out["R"] = normal_bf16(seed, TENSOR_IDS["R"], m, k, device=device)
    if scale_stream0 != 1.0:
        # power-of-two scale of stream 0: exact in bf16 (as if applied in fp32 before rounding)
        out["R"][:, :hs] = (out["R"][:, :hs].float() * scale_stream0).to(torch.bfloat16)
    out["y"] = normal_bf16(seed, TENSOR_IDS["y"], m, hs, device=device)
    inj = normal_bf16(seed, TENSOR_IDS["inj"], m, hc, device=device)
    if ld != hc:
        full = torch.zeros((m, ld), dtype=torch.bfloat16, device=device)
        full[:, :hc] = inj
        inj = full
    out["inj"] = inj
    out["ld_inj"] = ld
    if weights is None:
        weights = make_weights(shape, seed=seed, device=device, wnorm_full=wnorm_full,
                               wd_std=wd_std, wu_std=wu_std)
    out.update(weights)
    return out


def make_weights(shape: Shape = Shape(), *, seed: int = 0, device="cpu", wnorm_full: bool = False,
                 wd_std: float | None = None, wu_std: float | None = None) -> dict:
    hc, hs, r, k = shape.hc, shape.hs, shape.r, shape.k
    wlen = k if wnorm_full else hs
    sd = (1.0 / math.sqrt(k)) if wd_std is None else wd_std
    su = (1.0 / math.sqrt(r)) if wu_std is None else wu_std
    return {
        "wnorm": normal_bf16(seed, TENSOR_IDS["wnorm"], 1, wlen, std=0.1, device=device).reshape(wlen),
        "wd": normal_bf16(seed, TENSOR_IDS["wd"], r, k, std=sd, device=device),
        "wi": normal_bf16(seed, TENSOR_IDS["wi"], hc, k, std=sd, device=device),
        "wu": normal_bf16(seed, TENSOR_IDS["wu"], k, r, std=su, device=device),
    }


def fold_merged_weight(wd: torch.Tensor, wi: torch.Tensor, wnorm: torch.Tensor, n_pad: int,
                       hs: int) -> torch.Tensor:
    """Caller-side preparation of the merged down/inject weight [n_pad, K]:
    rows 0..r-1 = wd, rows r..r+HC-1 = wi, the rest zero, each column k scaled by
    (1 + wnorm[k mod HS]) (or wnorm[k] when wnorm is full width) in fp32 and
    rounded to bf16 (round-to-nearest-even)."""
    r, k = wd.shape
    hc = wi.shape[0]
    assert n_pad >= r + hc
    w = torch.zeros((n_pad, k), dtype=torch.float32, device=wd.device)
    w[:r] = wd.float()
    w[r:r + hc] = wi.float()
    wn = wnorm.float()
    if wn.numel() != k:
        wn = wn.repeat(k // wn.numel())
    w = w * (1.0 + wn).reshape(1, k)
    return w.to(torch.bfloat16)
