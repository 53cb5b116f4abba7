"""Python binding of the MI355X Hyper-Connection Gated Residual library.

The functions below carry the C ABI names of ``include/hcgr.h`` and only
marshal arguments (tensor pointers, sizes, the current HIP stream) to
``libhcgr.so``; every step of the op runs in the library's HIP kernels.
PyTorch provides device memory and streams. There is no fallback: if the
library is missing or cannot be loaded, every call raises.

``HCGR`` is a small convenience object over the same calls that allocates
outputs and the workspace with torch on the tensors' device.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhcgr.so")

HCGR_OK = 0
HCGR_ERR_INVALID_ARGUMENT = 1
HCGR_ERR_UNSUPPORTED = 2
HCGR_ERR_ALIASING = 3
HCGR_ERR_WORKSPACE_TOO_SMALL = 4
HCGR_ERR_HIP = 5
HCGR_WEIGHTS_SEPARATE = 0
HCGR_WEIGHTS_MERGED_FOLDED = 1
HCGR_PLAN_HEURISTIC = -1
HCGR_PLAN_SPLIT = 0
HCGR_PLAN_TILE = 3
HCGR_PLAN_FUSED = 4
HCGR_PLAN_PERSISTENT = 5
HCGR_SPLIT_VARIANTS = 13  # down-kernel variants of the decode plans (include/hcgr.h)
HCGR_WORKSPACE_COUNTER_BYTES = 131072
HCGR_DEFAULT_WAIT_POLLS = 1 << 20
HCGR_MAX_WAIT_POLLS = 1 << 24
PLAN_FIELDS = ("tokens", "kind", "down_variant", "streams_per_wg", "segments", "up_variant", "ranges")


class HcgrError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}: {detail}")


class hcgr_config(ctypes.Structure):
    _fields_ = [("hc", ctypes.c_int32), ("hs", ctypes.c_int32), ("r", ctypes.c_int32),
                ("eps", ctypes.c_float), ("wnorm_len", ctypes.c_int32),
                ("weight_layout", ctypes.c_int32), ("n_pad", ctypes.c_int32)]


class hcgr_plan_choice(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("kind", ctypes.c_int32), ("down_variant", ctypes.c_int32),
                ("streams_per_wg", ctypes.c_int32), ("segments", ctypes.c_int32), ("up_variant", ctypes.c_int32),
                ("ranges", ctypes.c_int32)]


def _choices_in(table):
    """A table (list of dicts with PLAN_FIELDS keys) as a ctypes array and its length."""
    table = list(table or [])
    arr = (hcgr_plan_choice * max(1, len(table)))()
    for i, e in enumerate(table):
        for f in PLAN_FIELDS:
            setattr(arr[i], f, int(e.get(f, 0)))
    return arr, len(table)


def _choice_out(c) -> dict:
    return {f: int(getattr(c, f)) for f in PLAN_FIELDS}


@dataclass(frozen=True)
class Config:
    hc: int = 4
    hs: int = 2560
    r: int = 320
    eps: float = 1e-6
    wnorm_len: int = 0          # 0 means hs
    weight_layout: int = HCGR_WEIGHTS_SEPARATE
    n_pad: int = 0

    def c(self) -> hcgr_config:
        return hcgr_config(self.hc, self.hs, self.r, self.eps, self.wnorm_len or self.hs,
                           self.weight_layout, self.n_pad)

    @property
    def k(self) -> int:
        return self.hc * self.hs

    @property
    def merged(self) -> bool:
        return self.weight_layout == HCGR_WEIGHTS_MERGED_FOLDED


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libhcgr.so (built by ``skinny_gemm_hcgr_amd.build``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m skinny_gemm_hcgr_amd.build` "
                           "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(path)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    CFG = ctypes.POINTER(hcgr_config)
    lib.hcgr_create.argtypes = [CFG, ctypes.c_int, ctypes.POINTER(P)]
    lib.hcgr_destroy.argtypes = [P]
    lib.hcgr_destroy.restype = None
    lib.hcgr_workspace_size.argtypes = [P, I64, ctypes.POINTER(SZ)]
    lib.hcgr_workspace_size_for.argtypes = [CFG, I64, ctypes.POINTER(SZ)]
    lib.hcgr_forward.argtypes = [P, P, P, P, I64, P, P, P, P, I64, P, P, P, I64, P, P, SZ, P]
    lib.hcgr_forward_timed.argtypes = [P, P, P, P, I64, P, P, P, P, I64, P, P, P, I64, P, P, SZ, P,
                                       ctypes.POINTER(P)]
    lib.hcgr_forward_noalloc.argtypes = [P, P, P, P, I64, P, P, P, P, I64, P, P, P, I64, P, P]
    lib.hcgr_noalloc_scratch_bytes.argtypes = []
    lib.hcgr_noalloc_scratch_bytes.restype = SZ
    lib.hcgr_validate.argtypes = [CFG, P, P, P, I64, P, P, P, P, I64, P, P, P, I64, P, P, SZ]
    lib.hcgr_combine.argtypes = [P, P, P, P, I64, I64, P, P]
    lib.hcgr_mix.argtypes = [P, P, P, P, P, P, I64, P, P, I64, P, P, SZ, P]
    lib.hcgr_validate_combine.argtypes = [CFG, P, P, P, I64, I64, P]
    lib.hcgr_validate_mix.argtypes = [CFG, P, P, P, P, P, I64, P, P, I64, P, P, SZ]
    lib.hcgr_describe_plan.argtypes = [CFG, I64, ctypes.c_char_p, SZ]
    PC = ctypes.POINTER(hcgr_plan_choice)
    lib.hcgr_plan_candidates.argtypes = [CFG, I64, PC, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)]
    lib.hcgr_plan_lookup.argtypes = [CFG, PC, ctypes.c_int32, I64, PC, ctypes.c_char_p, SZ]
    lib.hcgr_workspace_size_table.argtypes = [CFG, PC, ctypes.c_int32, I64, ctypes.POINTER(SZ)]
    lib.hcgr_set_plan_table.argtypes = [P, PC, ctypes.c_int32]
    lib.hcgr_set_wait_polls.argtypes = [P, ctypes.c_int32]
    lib.hcgr_status_string.argtypes = [ctypes.c_int]
    lib.hcgr_status_string.restype = ctypes.c_char_p
    lib.hcgr_last_error.argtypes = []
    lib.hcgr_last_error.restype = ctypes.c_char_p
    for name in ("hcgr_create", "hcgr_workspace_size", "hcgr_workspace_size_for", "hcgr_forward",
                 "hcgr_forward_timed", "hcgr_forward_noalloc", "hcgr_combine", "hcgr_mix", "hcgr_validate_combine",
                 "hcgr_validate_mix", "hcgr_validate", "hcgr_describe_plan", "hcgr_plan_candidates",
                 "hcgr_plan_lookup", "hcgr_workspace_size_table", "hcgr_set_plan_table", "hcgr_set_wait_polls"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().hcgr_status_string(int(status)).decode()


def last_error() -> str:
    return load_library().hcgr_last_error().decode()


def _check(status: int, where: str) -> int:
    if status != HCGR_OK:
        raise HcgrError(status, where, last_error())
    return status


def _p(t) -> int:
    """Device (or host) address of a tensor, an int address, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


# ------------------------------------------------------- C ABI, same names --
def hcgr_create(cfg: Config, device: int = 0) -> int:
    h = ctypes.c_void_p()
    c = cfg.c()
    _check(load_library().hcgr_create(ctypes.byref(c), int(device), ctypes.byref(h)), "hcgr_create")
    return h.value


def hcgr_destroy(handle: int) -> None:
    load_library().hcgr_destroy(handle)


def hcgr_workspace_size(handle: int, M: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().hcgr_workspace_size(handle, int(M), ctypes.byref(n)), "hcgr_workspace_size")
    return n.value


def hcgr_workspace_size_for(cfg: Config, M: int) -> int:
    n = ctypes.c_size_t()
    c = cfg.c()
    _check(load_library().hcgr_workspace_size_for(ctypes.byref(c), int(M), ctypes.byref(n)),
           "hcgr_workspace_size_for")
    return n.value


def hcgr_describe_plan(cfg: Config, M: int) -> str:
    buf = ctypes.create_string_buffer(1024)
    c = cfg.c()
    _check(load_library().hcgr_describe_plan(ctypes.byref(c), int(M), buf, len(buf)), "hcgr_describe_plan")
    return buf.value.decode()


def hcgr_plan_candidates(cfg: Config, M: int) -> list:
    """Every plan choice that can run cfg's shape at M tokens (dicts with PLAN_FIELDS)."""
    lib, c, n = load_library(), cfg.c(), ctypes.c_int32()
    _check(lib.hcgr_plan_candidates(ctypes.byref(c), int(M), None, 0, ctypes.byref(n)), "hcgr_plan_candidates")
    arr = (hcgr_plan_choice * max(1, n.value))()
    _check(lib.hcgr_plan_candidates(ctypes.byref(c), int(M), arr, n.value, ctypes.byref(n)), "hcgr_plan_candidates")
    return [_choice_out(arr[i]) for i in range(n.value)]


def hcgr_plan_lookup(cfg: Config, table, M: int):
    """(choice the table resolves M to, description of the resulting plan)."""
    c, (arr, n) = cfg.c(), _choices_in(table)
    out, buf = hcgr_plan_choice(), ctypes.create_string_buffer(1024)
    _check(load_library().hcgr_plan_lookup(ctypes.byref(c), arr, n, int(M), ctypes.byref(out), buf, len(buf)),
           "hcgr_plan_lookup")
    return _choice_out(out), buf.value.decode()


def hcgr_workspace_size_table(cfg: Config, table, M: int) -> int:
    c, (arr, n), b = cfg.c(), _choices_in(table), ctypes.c_size_t()
    _check(load_library().hcgr_workspace_size_table(ctypes.byref(c), arr, n, int(M), ctypes.byref(b)),
           "hcgr_workspace_size_table")
    return b.value


def hcgr_set_plan_table(handle: int, table) -> None:
    arr, n = _choices_in(table)
    _check(load_library().hcgr_set_plan_table(handle, arr, n), "hcgr_set_plan_table")


def hcgr_set_wait_polls(handle: int, polls: int) -> None:
    _check(load_library().hcgr_set_wait_polls(handle, int(polls)), "hcgr_set_wait_polls")


PLANS_DIR = os.path.join(_PKG, "plans")


def shipped_plan_table(cfg: Config):
    """Path of the tuned table shipped with the package for cfg (written by
    ``skinny_gemm_hcgr_amd.tune`` on an MI355X), or None."""
    name = f"hc{cfg.hc}_hs{cfg.hs}_r{cfg.r}" + ("_merged" if cfg.merged else "") + \
        ("_wnfull" if (cfg.wnorm_len or cfg.hs) != cfg.hs else "") + ".json"
    path = os.path.join(PLANS_DIR, name)
    return path if os.path.exists(path) else None


def load_plan_table(path: str, cfg: Config) -> list:
    """Entries of a tuned-plan JSON file (written by ``skinny_gemm_hcgr_amd.tune``);
    raises if the file was tuned for another configuration."""
    import json
    with open(path) as f:
        d = json.load(f)
    want = {"hc": cfg.hc, "hs": cfg.hs, "r": cfg.r, "wnorm_len": cfg.wnorm_len or cfg.hs,
            "weight_layout": cfg.weight_layout}
    got = {k: d.get("config", {}).get(k) for k in want}
    if got != want:
        raise ValueError(f"{path} was tuned for {got}, not {want}")
    return [{f: int(e[f]) for f in PLAN_FIELDS} for e in d["entries"]]


def _stream(stream, like):
    """Raw hipStream_t from an int, a torch stream, or None (torch's current
    stream on the device of the tensor ``like``)."""
    if stream is None:
        import torch
        dev = like.device if hasattr(like, "device") else None
        return torch.cuda.current_stream(dev).cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def hcgr_forward(handle, R, y, inj, ld_inj, wnorm, wd, wi, wu, M, R2, rrms, inj_next, ld_inj_next, x,
                 workspace, workspace_bytes, stream=None, *, check: bool = True) -> int:
    """Tensors (or raw addresses) in, status out; ``stream`` is a raw hipStream_t
    (an int), a torch stream, or None for torch's current stream on ``R``'s device."""
    stream = _stream(stream, R)
    st = load_library().hcgr_forward(handle, _p(R), _p(y), _p(inj), int(ld_inj), _p(wnorm), _p(wd), _p(wi),
                                     _p(wu), int(M), _p(R2), _p(rrms), _p(inj_next), int(ld_inj_next), _p(x),
                                     _p(workspace), int(workspace_bytes), stream)
    if check:
        _check(st, "hcgr_forward")
    return st


def hcgr_forward_timed(handle, R, y, inj, ld_inj, wnorm, wd, wi, wu, M, R2, rrms, inj_next, ld_inj_next, x,
                       workspace, workspace_bytes, stream, events) -> int:
    """``hcgr_forward`` plus 6 caller-owned hipEvent_t handles (ints): events
    2i and 2i+1 take the start and end of stage i's kernel (down/inject,
    reduction, up/mix)."""
    if not isinstance(stream, int):
        stream = stream.cuda_stream
    if len(events) != 6:
        raise ValueError("hcgr_forward_timed takes 6 events")
    ev = (ctypes.c_void_p * 6)(*events)
    st = load_library().hcgr_forward_timed(handle, _p(R), _p(y), _p(inj), int(ld_inj), _p(wnorm), _p(wd), _p(wi),
                                           _p(wu), int(M), _p(R2), _p(rrms), _p(inj_next), int(ld_inj_next), _p(x),
                                           _p(workspace), int(workspace_bytes), stream, ev)
    return _check(st, "hcgr_forward_timed")


def hcgr_forward_noalloc(handle, R, y, inj, ld_inj, wnorm, wd, wi, wu, M, R2, rrms, inj_next, ld_inj_next, x,
                         stream=None, *, check: bool = True) -> int:
    """``hcgr_forward`` on the library's own per-GPU scratch instead of a caller
    workspace (stream as in ``hcgr_forward``)."""
    stream = _stream(stream, R)
    st = load_library().hcgr_forward_noalloc(handle, _p(R), _p(y), _p(inj), int(ld_inj), _p(wnorm), _p(wd), _p(wi),
                                             _p(wu), int(M), _p(R2), _p(rrms), _p(inj_next), int(ld_inj_next),
                                             _p(x), stream)
    if check:
        _check(st, "hcgr_forward_noalloc")
    return st


def hcgr_noalloc_scratch_bytes() -> int:
    return int(load_library().hcgr_noalloc_scratch_bytes())


def hcgr_combine(handle, R, y, inj, ld_inj, M, R2, stream=None, *, check: bool = True) -> int:
    """(COMBINE) alone: R2 = R + y*iw (stream as in ``hcgr_forward``)."""
    st = load_library().hcgr_combine(handle, _p(R), _p(y), _p(inj), int(ld_inj), int(M), _p(R2),
                                     _stream(stream, R))
    if check:
        _check(st, "hcgr_combine")
    return st


def hcgr_mix(handle, R, wnorm, wd, wi, wu, M, rrms, inj_next, ld_inj_next, x, workspace, workspace_bytes,
             stream=None, *, check: bool = True) -> int:
    """Every step but COMBINE on a residual R taken as R2 (stream as in ``hcgr_forward``)."""
    st = load_library().hcgr_mix(handle, _p(R), _p(wnorm), _p(wd), _p(wi), _p(wu), int(M), _p(rrms),
                                 _p(inj_next), int(ld_inj_next), _p(x), _p(workspace), int(workspace_bytes),
                                 _stream(stream, R))
    if check:
        _check(st, "hcgr_mix")
    return st


def hcgr_validate_combine(cfg: Config, R, y, inj, ld_inj, M, R2) -> int:
    """Host-only checks of ``hcgr_combine``; returns the status code (does not raise)."""
    c = cfg.c()
    return load_library().hcgr_validate_combine(ctypes.byref(c), _p(R), _p(y), _p(inj), int(ld_inj), int(M),
                                                _p(R2))


def hcgr_validate_mix(cfg: Config, R, wnorm, wd, wi, wu, M, rrms, inj_next, ld_inj_next, x, workspace,
                      workspace_bytes) -> int:
    """Host-only checks of ``hcgr_mix``; returns the status code (does not raise)."""
    c = cfg.c()
    return load_library().hcgr_validate_mix(ctypes.byref(c), _p(R), _p(wnorm), _p(wd), _p(wi), _p(wu), int(M),
                                            _p(rrms), _p(inj_next), int(ld_inj_next), _p(x), _p(workspace),
                                            int(workspace_bytes))


def hcgr_validate(cfg: Config, R, y, inj, ld_inj, wnorm, wd, wi, wu, M, R2, rrms, inj_next, ld_inj_next, x,
                  workspace, workspace_bytes) -> int:
    """Host-only argument checks; returns the status code (does not raise)."""
    c = cfg.c()
    return load_library().hcgr_validate(ctypes.byref(c), _p(R), _p(y), _p(inj), int(ld_inj), _p(wnorm), _p(wd),
                                        _p(wi), _p(wu), int(M), _p(R2), _p(rrms), _p(inj_next),
                                        int(ld_inj_next), _p(x), _p(workspace), int(workspace_bytes))


def new_workspace(nbytes: int, device: int = 0):
    """A zero-filled device workspace of at least nbytes (the counter bytes at
    its start must be zero before the first call that uses it)."""
    import torch
    return torch.zeros(max(int(nbytes), HCGR_WORKSPACE_COUNTER_BYTES), dtype=torch.uint8, device=f"cuda:{device}")


# ------------------------------------------------------------ convenience --
class HCGR:
    """Handle + torch-allocated outputs/workspace around ``hcgr_forward``."""

    def __init__(self, cfg: Config = Config(), device: int = 0, plan_table=None):
        """``plan_table``: a tuned table (list of entries, or the path of a JSON
        file written by ``skinny_gemm_hcgr_amd.tune``), "shipped" for the table
        shipped with the package for cfg (the heuristic if there is none), or
        None for the heuristic."""
        self.cfg = cfg
        self.device = device
        self.handle = hcgr_create(cfg, device)
        self._ws = None
        if plan_table == "shipped":
            plan_table = shipped_plan_table(cfg)
        if plan_table is not None:
            self.set_plan_table(plan_table)

    def set_plan_table(self, table):
        if isinstance(table, str):
            table = load_plan_table(table, self.cfg)
        hcgr_set_plan_table(self.handle, table)
        self.table = list(table)
        self._ws = None  # the workspace bound may change

    def set_wait_polls(self, polls: int):
        hcgr_set_wait_polls(self.handle, polls)

    def describe(self, M: int) -> str:
        return hcgr_plan_lookup(self.cfg, getattr(self, "table", []), M)[1]

    def close(self):
        if self.handle:
            hcgr_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace(self, M: int):
        """A workspace for M tokens, zero-filled when allocated (the library
        keeps its counter bytes zero afterwards)."""
        n = hcgr_workspace_size(self.handle, M)
        if self._ws is None or self._ws.numel() < n:
            self._ws = new_workspace(n, self.device)
        return self._ws

    def alloc_outputs(self, M: int, ld_inj_next: int | None = None):
        import torch
        c = self.cfg
        dev = f"cuda:{self.device}"
        ld = c.hc if ld_inj_next is None else ld_inj_next
        packed = torch.zeros((M, ld), dtype=torch.bfloat16, device=dev)
        return {"R2": torch.empty((M, c.k), dtype=torch.bfloat16, device=dev),
                "rrms": torch.empty((M, c.hc), dtype=torch.float32, device=dev),
                "inj_next_buf": packed, "inj_next": packed[:, :c.hc], "ld_inj_next": ld,
                "x": torch.empty((M, c.hs), dtype=torch.bfloat16, device=dev)}

    def combine(self, R, y, inj, *, ld_inj: int | None = None, R2=None, stream=None):
        import torch
        M = R.shape[0]
        if R2 is None:
            R2 = torch.empty((M, self.cfg.k), dtype=torch.bfloat16, device=R.device)
        ld = inj.stride(0) if ld_inj is None else ld_inj
        hcgr_combine(self.handle, R, y, inj, ld, M, R2, stream)
        return R2

    def mix(self, R, wnorm, wd, wi, wu, *, out: dict | None = None, workspace=None, stream=None) -> dict:
        M = R.shape[0]
        if out is None:
            out = self.alloc_outputs(M)
        ws = self.workspace(M) if workspace is None else workspace
        hcgr_mix(self.handle, R, wnorm, wd, wi, wu, M, out["rrms"], out["inj_next"], out["ld_inj_next"],
                 out["x"], ws, ws.numel(), stream)
        return out

    def forward(self, R, y, inj, wnorm, wd, wi, wu, *, ld_inj: int | None = None, out: dict | None = None,
                workspace=None, stream=None) -> dict:
        M = R.shape[0]
        if out is None:
            out = self.alloc_outputs(M)
        ws = self.workspace(M) if workspace is None else workspace
        ld = inj.stride(0) if ld_inj is None else ld_inj
        hcgr_forward(self.handle, R, y, inj, ld, wnorm, wd, wi, wu, M, out["R2"], out["rrms"],
                     out["inj_next"], out["ld_inj_next"], out["x"], ws, ws.numel(), stream)
        return out
