"""Python face of the fp64 CPU oracle for the HCGR op (test infrastructure).

Only the test-suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It never touches the GPU library.

``forward`` follows ROCm/aiter pull request #5913 ("Two-stage Hyper-Connection
Gated Residual kernel", section "Technical Details": COMBINE, N, G1, G2, MIX,
INJ); the arithmetic lives in ``hcgr_oracle.c`` next to this file. ``combine``
and ``mix`` are the two parts that the same page's "PR Self-Review" section
lists as entry points of their own: COMBINE alone, and every other step on a
residual taken as R2 (no injection).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hcgr_oracle.c")
LIB_PATH = os.path.join(_HERE, "libhcgr_oracle.so")

__all__ = ["build", "load", "forward", "combine", "mix", "OracleConfig", "max_threads", "LIB_PATH"]


def build(src: str = _SRC, out: str = LIB_PATH, extra_flags=()) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP over tokens, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           *extra_flags, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class _Cfg(ctypes.Structure):
    _fields_ = [("hc", ctypes.c_int32), ("hs", ctypes.c_int32), ("r", ctypes.c_int32),
                ("wnorm_full", ctypes.c_int32), ("merged", ctypes.c_int32),
                ("n_pad", ctypes.c_int32), ("eps", ctypes.c_double)]


_LIBS: dict = {}


def load(path: str = LIB_PATH):
    """Load (building it first if absent) the oracle shared library at ``path``."""
    if path in _LIBS:
        return _LIBS[path]
    if not os.path.exists(path):
        if path != LIB_PATH:
            raise FileNotFoundError(path)
        build()
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.hcgr_oracle_forward.restype = ctypes.c_int
    lib.hcgr_oracle_forward.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int64, P, P, P,
                                        ctypes.c_int64, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                        ctypes.c_int]
    lib.hcgr_oracle_combine.restype = ctypes.c_int
    lib.hcgr_oracle_combine.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int64, P, P, P, ctypes.c_int64,
                                        P, ctypes.c_int]
    lib.hcgr_oracle_mix.restype = ctypes.c_int
    lib.hcgr_oracle_mix.argtypes = [ctypes.POINTER(_Cfg), ctypes.c_int64, P, P, P, P, P, P, P, P,
                                    P, P, P, P, P, ctypes.c_int]
    lib.hcgr_oracle_max_threads.restype = ctypes.c_int
    _LIBS[path] = lib
    return lib


def max_threads(path: str = LIB_PATH) -> int:
    return int(load(path).hcgr_oracle_max_threads())


@dataclass(frozen=True)
class OracleConfig:
    hc: int = 4
    hs: int = 2560
    r: int = 320
    eps: float = 1e-6
    wnorm_full: bool = False
    merged: bool = False
    n_pad: int = 0

    @property
    def k(self) -> int:
        return self.hc * self.hs


def _u16(a) -> np.ndarray:
    """bf16 input as a contiguous numpy uint16 array (accepts numpy uint16 or a torch bf16 tensor)."""
    if isinstance(a, np.ndarray):
        assert a.dtype == np.uint16, a.dtype
        return np.ascontiguousarray(a)
    import torch  # local: the oracle itself does not need torch
    assert a.dtype == torch.bfloat16, a.dtype
    return a.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)


def _ptr(a) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data) if a is not None else ctypes.c_void_p(0)


def forward(cfg: OracleConfig, R, y, inj, wnorm, wd, wi, wu, *, ld_inj: int | None = None,
            threads: int = 0, debug: bool = False, lib_path: str = LIB_PATH) -> dict:
    """Run the oracle on M tokens. ``R`` [M,K], ``y`` [M,HS], ``inj`` [M,ld_inj];
    ``wd`` is Wd [r,K] (or the folded Wm [n_pad,K] when ``cfg.merged``), ``wi`` is
    Wi [HC,K] (ignored when merged), ``wu`` is Wu [K,r]. Returns fp64 numpy arrays
    ``R2`` [M,K], ``rrms`` [M,HC], ``inj_next`` [M,HC], ``x`` [M,HS]; with
    ``debug`` also ``xn``, ``lora``, ``h``, ``gate``, ``G``."""
    lib = load(lib_path)
    R, y, inj, wnorm, wd, wu = map(_u16, (R, y, inj, wnorm, wd, wu))
    wi = None if cfg.merged else _u16(wi)
    M = R.shape[0] if R.ndim == 2 else 0
    K, HS, HC, r = cfg.k, cfg.hs, cfg.hc, cfg.r
    ld = HC if ld_inj is None else int(ld_inj)
    assert R.size == M * K and y.size == M * HS
    if M:
        assert inj.size >= (M - 1) * ld + HC
    assert wnorm.size == (K if cfg.wnorm_full else HS)
    assert wd.size == (cfg.n_pad if cfg.merged else r) * K and wu.size == K * r
    if wi is not None:
        assert wi.size == HC * K
    out = {"R2": np.empty((M, K)), "rrms": np.empty((M, HC)), "inj_next": np.empty((M, HC)),
           "x": np.empty((M, HS))}
    dbg_names = ("xn", "lora", "h", "gate", "G")
    if debug:
        out.update({"xn": np.empty((M, K)), "lora": np.empty((M, r)), "h": np.empty((M, r)),
                    "gate": np.empty((M, K)), "G": np.empty((M, K))})
    c = _Cfg(HC, HS, r, int(cfg.wnorm_full), int(cfg.merged), int(cfg.n_pad), float(cfg.eps))
    st = lib.hcgr_oracle_forward(ctypes.byref(c), M, _ptr(R), _ptr(y), _ptr(inj), ld, _ptr(wnorm),
                                 _ptr(wd), _ptr(wi), _ptr(wu), _ptr(out["R2"]), _ptr(out["rrms"]),
                                 _ptr(out["inj_next"]), _ptr(out["x"]),
                                 *[_ptr(out.get(n)) for n in dbg_names], int(threads))
    if st != 0:
        raise RuntimeError(f"hcgr_oracle_forward failed with status {st}")
    return out


def _cfg(cfg: OracleConfig) -> _Cfg:
    return _Cfg(cfg.hc, cfg.hs, cfg.r, int(cfg.wnorm_full), int(cfg.merged), int(cfg.n_pad), float(cfg.eps))


def combine(cfg: OracleConfig, R, y, inj, *, ld_inj: int | None = None, threads: int = 0,
            lib_path: str = LIB_PATH) -> dict:
    """(COMBINE) alone on M tokens: ``R`` [M,K], ``y`` [M,HS], ``inj`` [M,ld_inj]
    -> fp64 ``R2`` [M,K]."""
    lib = load(lib_path)
    R, y, inj = map(_u16, (R, y, inj))
    M = R.shape[0] if R.ndim == 2 else 0
    K, HS, HC = cfg.k, cfg.hs, cfg.hc
    ld = HC if ld_inj is None else int(ld_inj)
    assert R.size == M * K and y.size == M * HS
    if M:
        assert inj.size >= (M - 1) * ld + HC
    out = {"R2": np.empty((M, K))}
    st = lib.hcgr_oracle_combine(ctypes.byref(_cfg(cfg)), M, _ptr(R), _ptr(y), _ptr(inj), ld,
                                 _ptr(out["R2"]), int(threads))
    if st != 0:
        raise RuntimeError(f"hcgr_oracle_combine failed with status {st}")
    return out


def mix(cfg: OracleConfig, R, wnorm, wd, wi, wu, *, threads: int = 0, debug: bool = False,
        lib_path: str = LIB_PATH) -> dict:
    """Every step but COMBINE on M tokens whose residual ``R`` [M,K] is taken as
    R2: fp64 ``rrms`` [M,HC], ``inj_next`` [M,HC], ``x`` [M,HS] (with ``debug``
    also ``xn``, ``lora``, ``h``, ``gate``, ``G``). Weights as in ``forward``."""
    lib = load(lib_path)
    R, wnorm, wd, wu = map(_u16, (R, wnorm, wd, wu))
    wi = None if cfg.merged else _u16(wi)
    M = R.shape[0] if R.ndim == 2 else 0
    K, HS, HC, r = cfg.k, cfg.hs, cfg.hc, cfg.r
    assert R.size == M * K
    assert wnorm.size == (K if cfg.wnorm_full else HS)
    assert wd.size == (cfg.n_pad if cfg.merged else r) * K and wu.size == K * r
    if wi is not None:
        assert wi.size == HC * K
    out = {"rrms": np.empty((M, HC)), "inj_next": np.empty((M, HC)), "x": np.empty((M, HS))}
    dbg_names = ("xn", "lora", "h", "gate", "G")
    if debug:
        out.update({"xn": np.empty((M, K)), "lora": np.empty((M, r)), "h": np.empty((M, r)),
                    "gate": np.empty((M, K)), "G": np.empty((M, K))})
    st = lib.hcgr_oracle_mix(ctypes.byref(_cfg(cfg)), M, _ptr(R), _ptr(wnorm), _ptr(wd), _ptr(wi),
                             _ptr(wu), _ptr(out["rrms"]), _ptr(out["inj_next"]), _ptr(out["x"]),
                             *[_ptr(out.get(n)) for n in dbg_names], int(threads))
    if st != 0:
        raise RuntimeError(f"hcgr_oracle_mix failed with status {st}")
    return out
