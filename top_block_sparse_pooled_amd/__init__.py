"""Top-p block-sparse attention for MI355X (gfx950): thin Python binding of libfvattn.

Every step of the path runs in the HIP kernels of libfvattn.so; this module only
marshals arguments: it checks tensor shapes/dtypes, allocates outputs and workspaces
with torch (device memory), and passes raw pointers plus the current HIP stream to
the C ABI declared in include/fvattn.h.  There is no CPU fallback: if the library
is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

__all__ = [
    "FvAttnError", "Csr", "lib", "version", "csr_max_nnz", "route_ws_bytes", "attn_ws_bytes",
    "pool", "route", "worklist", "sparse_attn", "attn_plan", "attn_run", "SCHED", "ws_status", "plan_worklist",
    "sparse_attn_noalloc", "NOALLOC_MAX_ROWS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfvattn.so")

BF16, F32 = 0, 1
NOALLOC_MAX_ROWS = 262144   # FVATTN_NOALLOC_MAX_ROWS
SCHED = {"default": -1, "lpt": 0, "identity": 1, "head_lpt": 2, "xcd": 3, "rlb": 4, "head_desc": 5}
STATUS = {"select_nocross": 1, "plan_mismatch": 2}
ROUTE_MODES = {"topp": 0, "topk": 1}


class FvAttnError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: error {code} ({_strerror(code)})")
        self.code = code


class _CsrC(ctypes.Structure):
    _fields_ = [("bh", ctypes.c_int32), ("n", ctypes.c_int32), ("block_q", ctypes.c_int32),
                ("block_k", ctypes.c_int32), ("nqb", ctypes.c_int32), ("nkb", ctypes.c_int32),
                ("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p), ("capacity", ctypes.c_int64),
                ("head_load", ctypes.c_void_p)]


class _OptsC(ctypes.Structure):
    _fields_ = [("schedule", ctypes.c_int32), ("grid", ctypes.c_int32), ("trace", ctypes.c_void_p),
                ("trace_cap", ctypes.c_int64), ("out_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class _RouteOptsC(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("topk", ctypes.c_int32), ("p", ctypes.c_double),
                ("k_min", ctypes.c_int32), ("k_max", ctypes.c_int32), ("window", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class _SasaOptsC(ctypes.Structure):
    _fields_ = [("groups", ctypes.c_int32), ("critical", ctypes.c_int32), ("alpha", ctypes.c_double),
                ("tau", ctypes.c_double), ("added", ctypes.c_void_p)]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libfvattn.so (built in-tree by __graft_entry__.build / hipbuild.py)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m top_block_sparse_pooled_amd.hipbuild`")
        L = ctypes.CDLL(LIB_PATH)
        i32, i64, vp, sz, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_double
        L.fvattn_version.restype = i32
        L.fvattn_strerror.restype = ctypes.c_char_p
        L.fvattn_strerror.argtypes = [i32]
        L.fvattn_csr_max_nnz.restype = i64
        L.fvattn_csr_max_nnz.argtypes = [i32] * 5
        L.fvattn_route_ws_bytes.restype = sz
        L.fvattn_route_ws_bytes.argtypes = [i32] * 6
        L.fvattn_attn_ws_bytes.restype = sz
        L.fvattn_attn_ws_bytes.argtypes = [i32] * 7
        L.fvattn_pool.restype = i32
        L.fvattn_pool.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp]
        L.fvattn_route.restype = i32
        L.fvattn_route.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, dbl,
                                   ctypes.POINTER(_CsrC), vp, sz, vp]
        L.fvattn_route_ex.restype = i32
        L.fvattn_route_ex.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(_RouteOptsC),
                                      ctypes.POINTER(_CsrC), vp, sz, vp]
        L.fvattn_route_sasa_ws_bytes.restype = sz
        L.fvattn_route_sasa_ws_bytes.argtypes = [i32] * 7
        L.fvattn_route_sasa.restype = i32
        L.fvattn_route_sasa.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(_RouteOptsC),
                                        ctypes.POINTER(_SasaOptsC), ctypes.POINTER(_CsrC), vp, sz, vp]
        L.fvattn_worklist_ws_bytes.restype = sz
        L.fvattn_worklist_ws_bytes.argtypes = [i32]
        L.fvattn_worklist.restype = i32
        L.fvattn_worklist.argtypes = [ctypes.POINTER(_CsrC), i32, i32, vp, vp, sz, vp]
        L.fvattn_ws_status.restype = i32
        L.fvattn_ws_status.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_uint32), vp]
        L.fvattn_attn_plan.restype = i32
        L.fvattn_attn_plan.argtypes = [vp, i32, i32, i32, i32, i32, ctypes.POINTER(_CsrC), i32, vp, sz, vp]
        L.fvattn_attn_run.restype = i32
        L.fvattn_attn_run.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.POINTER(_CsrC),
                                      ctypes.POINTER(_OptsC), vp, sz, vp]
        L.fvattn_sparse_attn_noalloc.restype = i32
        L.fvattn_sparse_attn_noalloc.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.POINTER(_CsrC),
                                                 ctypes.POINTER(_OptsC), vp]
        L.fvattn_sparse_attn.restype = i32
        L.fvattn_sparse_attn.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, ctypes.POINTER(_CsrC),
                                         ctypes.POINTER(_OptsC), vp, sz, vp]
        _LIB = L
    return _LIB


def _strerror(code: int) -> str:
    try:
        return lib().fvattn_strerror(code).decode()
    except Exception:  # pragma: no cover - library missing
        return "?"


def _check(rc: int, what: str):
    if rc != 0:
        raise FvAttnError(rc, what)


def version() -> int:
    return lib().fvattn_version()


def csr_max_nnz(B, H, N, block_q, block_k) -> int:
    return lib().fvattn_csr_max_nnz(B, H, N, block_q, block_k)


def route_ws_bytes(B, H, N, d, block_q, block_k) -> int:
    return lib().fvattn_route_ws_bytes(B, H, N, d, block_q, block_k)


def attn_ws_bytes(B, H, N, d, dtype_code, block_q, block_k) -> int:
    return lib().fvattn_attn_ws_bytes(B, H, N, d, dtype_code, block_q, block_k)


# ------------------------------------------------------------------------ torch side
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}: use bfloat16 or float32")


def _stream(dev):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check_qkv(*ts):
    t0 = ts[0]
    if t0.dim() != 4:
        raise ValueError("tensors must be [B, H, N, d]")
    for t in ts:
        if t.shape != t0.shape or t.dtype != t0.dtype or t.device != t0.device:
            raise ValueError("q/k/v must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if t.device.type != "cuda":
            raise ValueError("tensors must live on the GPU")


@dataclasses.dataclass
class Csr:
    """Kept key blocks per (batch*head, query block) row, on the device (int32)."""
    row_ptr: "object"
    col_idx: "object"
    head_load: "object"
    bh: int
    n: int
    block_q: int
    block_k: int
    nqb: int
    nkb: int

    @property
    def rows(self) -> int:
        return self.bh * self.nqb

    def c(self) -> _CsrC:
        return _CsrC(self.bh, self.n, self.block_q, self.block_k, self.nqb, self.nkb,
                     self.row_ptr.data_ptr(), self.col_idx.data_ptr(), self.col_idx.numel(),
                     self.head_load.data_ptr())

    @classmethod
    def empty(cls, B, H, N, block_q, block_k, device):
        torch = _torch()
        cap = csr_max_nnz(B, H, N, block_q, block_k)
        if cap < 0:
            raise FvAttnError(int(cap), "csr_max_nnz")
        nqb, nkb = -(-N // block_q), -(-N // block_k)
        i32 = torch.int32
        return cls(torch.empty(B * H * nqb + 1, dtype=i32, device=device),
                   torch.empty(max(cap, 1), dtype=i32, device=device),
                   torch.empty(B * H, dtype=i32, device=device), B * H, N, block_q, block_k, nqb, nkb)

    @classmethod
    def from_host(cls, row_ptr, col_idx, head_load, bh, n, block_q, block_k, device):
        """Upload a CSR built elsewhere (for example by a reference implementation)."""
        torch = _torch()
        nqb, nkb = -(-n // block_q), -(-n // block_k)
        t = lambda a: torch.as_tensor(a, dtype=torch.int32).to(device)
        ci = t(col_idx) if len(col_idx) else torch.zeros(1, dtype=torch.int32, device=device)
        return cls(t(row_ptr), ci, t(head_load), bh, n, block_q, block_k, nqb, nkb)

    def nnz(self) -> int:
        return int(self.row_ptr[-1].item())


def pool(x, block: int):
    """Mean over the real tokens of each block: x [B, H, N, d] -> float64 [B, H, nb, d]."""
    torch = _torch()
    _check_qkv(x)
    B, H, N, d = x.shape
    nb = -(-N // block)
    out = torch.empty(B, H, nb, d, dtype=torch.float64, device=x.device)
    _check(lib().fvattn_pool(x.data_ptr(), B * H, N, d, _dtype_code(x), block, out.data_ptr(),
                             _stream(x.device)), "fvattn_pool")
    return out


def route(q, k, block_q: int, block_k: int, p: float = 0.9, csr: Optional[Csr] = None, ws=None,
          mode: str = "topp", topk: int = 0, k_min: int = 1, k_max: int = 0, window: int = 0) -> Csr:
    """Top-p routing (or a variant: mode="topk" with topk, a [k_min, k_max] clamp of the
    Top-p count, a local window) -> Csr.  `csr` / `ws` may be preallocated (reused)."""
    torch = _torch()
    _check_qkv(q, k)
    B, H, N, d = q.shape
    if csr is None:
        csr = Csr.empty(B, H, N, block_q, block_k, q.device)
    need = route_ws_bytes(B, H, N, d, block_q, block_k)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    c = csr.c()
    if mode == "topp" and k_min == 1 and k_max == 0 and window == 0:
        _check(lib().fvattn_route(q.data_ptr(), k.data_ptr(), B, H, N, d, _dtype_code(q), block_q, block_k,
                                  float(p), ctypes.byref(c), ws.data_ptr(), ws.numel(), _stream(q.device)),
               "fvattn_route")
    else:
        if mode not in ROUTE_MODES:
            raise ValueError(f"mode must be one of {sorted(ROUTE_MODES)}")
        o = _RouteOptsC(ROUTE_MODES[mode], int(topk), float(p), int(k_min), int(k_max), int(window), 0)
        _check(lib().fvattn_route_ex(q.data_ptr(), k.data_ptr(), B, H, N, d, _dtype_code(q), block_q, block_k,
                                     ctypes.byref(o), ctypes.byref(c), ws.data_ptr(), ws.numel(),
                                     _stream(q.device)),
               "fvattn_route_ex")
    csr.bh, csr.n, csr.block_q, csr.block_k, csr.nqb, csr.nkb = c.bh, c.n, c.block_q, c.block_k, c.nqb, c.nkb
    return csr


def route_sasa(q, k, block_q: int, block_k: int, p: float = 0.9, groups: int = 8, alpha: float = 0.5,
               tau: float = 0.0, critical: int = 0, csr: Optional[Csr] = None, ws=None, added=None,
               mode: str = "topp", topk: int = 0, k_min: int = 1, k_max: int = 0, window: int = 0) -> Csr:
    """Routing (Top-p or a variant) followed by SASA over `groups` contiguous head groups ->
    Csr of the augmented kept sets.  `added` (optional int32 tensor [groups]) receives the
    blocks added per group."""
    torch = _torch()
    _check_qkv(q, k)
    B, H, N, d = q.shape
    if mode not in ROUTE_MODES:
        raise ValueError(f"mode must be one of {sorted(ROUTE_MODES)}")
    if csr is None:
        csr = Csr.empty(B, H, N, block_q, block_k, q.device)
    need = lib().fvattn_route_sasa_ws_bytes(B, H, N, d, block_q, block_k, int(groups))
    if need == 0:
        raise ValueError("invalid shape or group count for SASA")
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    if added is not None and (added.dtype != torch.int32 or added.numel() < groups or not added.is_cuda):
        raise ValueError("added must be a CUDA int32 tensor with at least `groups` elements")
    ro = _RouteOptsC(ROUTE_MODES[mode], int(topk), float(p), int(k_min), int(k_max), int(window), 0)
    so = _SasaOptsC(int(groups), int(critical), float(alpha), float(tau),
                    added.data_ptr() if added is not None else None)
    c = csr.c()
    _check(lib().fvattn_route_sasa(q.data_ptr(), k.data_ptr(), B, H, N, d, _dtype_code(q), block_q, block_k,
                                   ctypes.byref(ro), ctypes.byref(so), ctypes.byref(c), ws.data_ptr(), ws.numel(),
                                   _stream(q.device)),
           "fvattn_route_sasa")
    csr.bh, csr.n, csr.block_q, csr.block_k, csr.nqb, csr.nkb = c.bh, c.n, c.block_q, c.block_k, c.nqb, c.nkb
    return csr


def worklist(csr: Csr, schedule: str = "lpt", G: int = 1, with_control: bool = False):
    """Device-built work list: a permutation of the units (G adjacent query blocks of one head;
    G = 1: CSR rows) in the given order.  with_control: also return the 64-word control block
    (per-XCD queue starts at words 16..24)."""
    torch = _torch()
    units = csr.bh * -(-csr.nqb // G)
    wl = torch.empty(units, dtype=torch.int32, device=csr.row_ptr.device)
    need = lib().fvattn_worklist_ws_bytes(csr.rows)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=wl.device)
    c = csr.c()
    _check(lib().fvattn_worklist(ctypes.byref(c), SCHED[schedule], int(G), wl.data_ptr(), ws.data_ptr(), ws.numel(),
                                 _stream(wl.device)), "fvattn_worklist")
    return (wl, ws[:256].view(torch.int32)) if with_control else wl


def ws_status(ws, which: str) -> int:
    """Status word (FVATTN_STATUS_* bits) that the last call left in a routing ("route") or
    attention ("attn") workspace; synchronises the current stream."""
    out = ctypes.c_uint32(0)
    _check(lib().fvattn_ws_status(ws.data_ptr(), {"route": 0, "attn": 1}[which], ctypes.byref(out),
                                  _stream(ws.device)), "fvattn_ws_status")
    return int(out.value)


def _trace_arg(trace):
    """(pointer, capacity in uint64 elements) of an optional int64/uint64 device trace tensor."""
    torch = _torch()
    if trace is None:
        return None, 0
    if trace.dtype not in (torch.int64, getattr(torch, "uint64", torch.int64)) or not trace.is_cuda \
            or not trace.is_contiguous():
        raise ValueError("trace must be a contiguous int64 CUDA tensor")
    return trace.data_ptr(), trace.numel()


def sparse_attn(q, k, v, csr: Csr, schedule: str = "default", grid: int = 0, trace=None, out=None, ws=None,
                out_dtype=None):
    """Block-sparse attention over the CSR's kept blocks -> o [B, H, N, d].
    out_dtype: None (dtype of q) or torch.float32 (accumulator precision, for bf16 inputs)."""
    torch = _torch()
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    odt = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(q.shape, dtype=odt, device=q.device)
    if out.dtype != odt or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, H, N, d] tensor of the output dtype")
    need = attn_ws_bytes(B, H, N, d, _dtype_code(q), csr.block_q, csr.block_k)
    if ws is None:
        ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    tp, tcap = _trace_arg(trace)
    opts = _OptsC(SCHED[schedule], grid, tp, tcap, -1 if odt == q.dtype else _dtype_code(out), 0)
    c = csr.c()
    _check(lib().fvattn_sparse_attn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, d,
                                    _dtype_code(q), ctypes.byref(c), ctypes.byref(opts), ws.data_ptr(),
                                    ws.numel(), _stream(q.device)), "fvattn_sparse_attn")
    return out


def sparse_attn_noalloc(q, k, v, csr: Csr, schedule: str = "default", grid: int = 0, trace=None, out=None,
                        out_dtype=None):
    """fvattn_sparse_attn_noalloc: as sparse_attn, with the plan in the library's static device
    scratch instead of a workspace (B*H*nqb <= NOALLOC_MAX_ROWS; calls on one GPU must not overlap)."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    out, odc = _attn_out(q, out, out_dtype)
    tp, tcap = _trace_arg(trace)
    opts = _OptsC(SCHED[schedule], grid, tp, tcap, odc, 0)
    c = csr.c()
    _check(lib().fvattn_sparse_attn_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, d,
                                            _dtype_code(q), ctypes.byref(c), ctypes.byref(opts), _stream(q.device)),
           "fvattn_sparse_attn_noalloc")
    return out


def _attn_out(q, out, out_dtype):
    torch = _torch()
    odt = q.dtype if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty(q.shape, dtype=odt, device=q.device)
    if out.dtype != odt or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, H, N, d] tensor of the output dtype")
    return out, (-1 if odt == q.dtype else _dtype_code(out))


def attn_ws(q, csr: Csr):
    torch = _torch()
    B, H, N, d = q.shape
    need = attn_ws_bytes(B, H, N, d, _dtype_code(q), csr.block_q, csr.block_k)
    return torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)


def attn_plan(v, csr: Csr, ws, schedule: str = "default"):
    """Work list of the CSR rows into ws (v supplies the shape only); see fvattn_attn_plan."""
    _check_qkv(v)
    B, H, N, d = v.shape
    c = csr.c()
    _check(lib().fvattn_attn_plan(v.data_ptr(), B, H, N, d, _dtype_code(v), ctypes.byref(c), SCHED[schedule],
                                  ws.data_ptr(), ws.numel(), _stream(v.device)), "fvattn_attn_plan")


def attn_run(q, k, v, csr: Csr, ws, out=None, out_dtype=None, grid: int = 0, trace=None):
    """The attention kernel alone on a plan held in ws; see fvattn_attn_run."""
    _check_qkv(q, k, v)
    B, H, N, d = q.shape
    out, odc = _attn_out(q, out, out_dtype)
    tp, tcap = _trace_arg(trace)
    opts = _OptsC(0, grid, tp, tcap, odc, 0)
    c = csr.c()
    _check(lib().fvattn_attn_run(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, d,
                                 _dtype_code(q), ctypes.byref(c), ctypes.byref(opts), ws.data_ptr(), ws.numel(),
                                 _stream(q.device)), "fvattn_attn_run")
    return out


def plan_worklist(csr: Csr, ws, units: int):
    """The work list that fvattn_attn_plan left in an attention workspace (first `units`
    entries, after the 256-byte control block)."""
    torch = _torch()
    return ws[256:256 + 4 * units].view(torch.int32)
