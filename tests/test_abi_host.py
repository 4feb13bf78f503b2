"""C-ABI checks that need no GPU: the library loads, exports every function the header
declares, and every validation path returns its documented code before anything is
enqueued (all calls below fail validation, so no kernel is ever launched)."""
import ctypes
import math
import os
import re

import pytest

import top_block_sparse_pooled_amd as fv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fvattn.h")

OK, INVALID, UNSUPPORTED, CAPACITY, WORKSPACE, OVERFLOW, HIP, MISMATCH, SCRATCH = 0, -1, -2, -3, -4, -5, -6, -7, -8
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call here fails validation first

# Fake device pointers must never reach a real launch: run these only where no GPU is visible.
def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


pytestmark = pytest.mark.skipif(_gpu_visible(), reason="host-only validation tests pass fake pointers")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fv.LIB_PATH):
        pytest.fail("libfvattn.so is not built (run __graft_entry__.build())")
    return fv.lib()


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fvattn_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert {"fvattn_route", "fvattn_sparse_attn", "fvattn_pool", "fvattn_worklist"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"missing export {n}"


def test_version_and_strerror(L):
    assert L.fvattn_version() == 10100
    for code in (OK, INVALID, UNSUPPORTED, CAPACITY, WORKSPACE, OVERFLOW, HIP, MISMATCH, SCRATCH):
        s = L.fvattn_strerror(code).decode()
        assert s and s != "unknown error code"
    assert L.fvattn_strerror(42).decode() == "unknown error code"


def test_sizes(L):
    assert L.fvattn_csr_max_nnz(1, 40, 32760, 64, 64) == 40 * 512 * 512
    assert L.fvattn_csr_max_nnz(1, 40, 75600, 128, 64) == 40 * 591 * 1182
    assert L.fvattn_csr_max_nnz(1, 1, 100, 48, 64) == UNSUPPORTED
    # pooled K in float64 (the query blocks are pooled inside the select kernel) + counts and masks
    assert L.fvattn_route_ws_bytes(1, 40, 32760, 128, 64, 64) > 40 * 512 * 128 * 8
    assert L.fvattn_route_ws_bytes(1, 40, 32760, 96, 64, 64) == 0
    bf = L.fvattn_attn_ws_bytes(1, 40, 32760, 128, 0, 64, 64)
    bf32 = L.fvattn_attn_ws_bytes(1, 40, 32760, 128, 0, 64, 32)
    f32 = L.fvattn_attn_ws_bytes(1, 40, 32760, 128, 1, 64, 64)
    # the work list and counters only: v is read as given for either key block size
    assert bf32 == bf == f32 >= 4 * 40 * 512 > 0
    assert L.fvattn_attn_ws_bytes(1, 40, 32760, 128, 7, 64, 64) == 0


def _csr(bh=2, n=1024, bq=64, bk=64, cap=None):
    nqb, nkb = -(-n // bq), -(-n // bk)
    c = fv._CsrC(bh, n, bq, bk, nqb, nkb, 0x2000, 0x3000, cap if cap is not None else bh * nqb * nkb, 0x4000)
    return c


def _route(L, B=1, H=2, N=1024, d=64, dt=0, bq=64, bk=64, p=0.9, csr=None, ws=FAKE, ws_bytes=1 << 40,
           q=FAKE, k=FAKE):
    c = csr if csr is not None else _csr(B * H, N, bq, bk)
    return L.fvattn_route(q, k, B, H, N, d, dt, bq, bk, p, ctypes.byref(c) if c is not False else None,
                          ws, ws_bytes, None)


@pytest.mark.parametrize("p", [0.0, -0.1, 1.0000001, 1.5, math.nan, -math.inf])
def test_route_rejects_bad_p(L, p):
    assert _route(L, p=p) == INVALID


@pytest.mark.parametrize("kw,code", [
    (dict(d=96), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(bq=48), UNSUPPORTED),
    (dict(bk=128), UNSUPPORTED), (dict(dt=5), UNSUPPORTED), (dict(B=0), INVALID), (dict(H=-1), INVALID),
    (dict(N=0), INVALID), (dict(q=None), INVALID), (dict(k=None), INVALID), (dict(ws=None), INVALID),
    (dict(csr=False), INVALID), (dict(N=262145, bk=64), UNSUPPORTED), (dict(N=131073, bk=32), UNSUPPORTED),
])
def test_route_validation(L, kw, code):
    assert _route(L, **kw) == code


def test_route_overflow(L):
    c = _csr(60000, 81920, 32, 64)
    assert _route(L, B=2000, H=30, N=81920, bq=32, bk=64, csr=c) == OVERFLOW


def test_route_capacity_and_workspace(L):
    c = _csr(2, 1024, 64, 64, cap=2 * 16 * 16 - 1)
    assert _route(L, csr=c) == CAPACITY
    need = L.fvattn_route_ws_bytes(1, 2, 1024, 64, 64, 64)
    assert _route(L, ws_bytes=need - 1) == WORKSPACE
    c = _csr()
    c.row_ptr = None
    assert _route(L, csr=c) == INVALID


def _attn(L, B=1, H=2, N=1024, d=64, dt=0, csr=None, opts=None, ws_bytes=1 << 40, v=FAKE):
    c = csr if csr is not None else _csr(2, 1024)   # always describes B*H=2, N=1024
    return L.fvattn_sparse_attn(FAKE, FAKE, v, FAKE, B, H, N, d, dt, ctypes.byref(c),
                                ctypes.byref(opts) if opts is not None else None, FAKE, ws_bytes, None)


def test_attn_validation(L):
    assert _attn(L, dt=3) == UNSUPPORTED
    assert _attn(L, v=None) == INVALID
    assert _attn(L, N=1000) == MISMATCH                     # csr built for N=1024
    assert _attn(L, H=3) == MISMATCH
    assert _attn(L, opts=fv._OptsC(9, 0, None, 0, -1, 0)) == INVALID
    assert _attn(L, opts=fv._OptsC(0, -4, None, 0, -1, 0)) == INVALID
    assert _attn(L, opts=fv._OptsC(0, 0, None, 0, 7, 0)) == UNSUPPORTED          # unknown output dtype
    assert _attn(L, dt=1, opts=fv._OptsC(0, 0, None, 0, 0, 0)) == UNSUPPORTED  # fp32 inputs, bf16 output
    # trace capacity: 4 records per unit (bf16: units of 128 query rows = 2 query blocks of 64 -> 2 * 8 units)
    assert _attn(L, opts=fv._OptsC(0, 0, FAKE, 4 * 16 - 1, -1, 0)) == INVALID
    assert _attn(L, opts=fv._OptsC(0, 0, FAKE, 4 * 16 - 1, -1, 0), ws_bytes=1) == WORKSPACE  # ws checked first
    assert _attn(L, dt=1, opts=fv._OptsC(0, 0, FAKE, 4 * 32 - 1, -1, 0)) == INVALID  # f32: one unit per row
    need = L.fvattn_attn_ws_bytes(1, 2, 1024, 64, 0, 64, 64)
    assert _attn(L, ws_bytes=need - 1) == WORKSPACE
    assert L.fvattn_sparse_attn(FAKE, FAKE, FAKE, FAKE, 1, 2, 1024, 64, 0, None, None, FAKE, 1 << 40,
                                None) == INVALID


def test_plan_run_validation(L):
    c = _csr(2, 1024)
    need = L.fvattn_attn_ws_bytes(1, 2, 1024, 64, 0, 64, 64)
    assert L.fvattn_attn_plan(FAKE, 1, 2, 1024, 64, 0, ctypes.byref(c), 9, FAKE, need, None) == INVALID
    assert L.fvattn_attn_plan(FAKE, 1, 2, 1024, 64, 0, ctypes.byref(c), 0, FAKE, need - 1, None) == WORKSPACE
    assert L.fvattn_attn_plan(FAKE, 1, 2, 1000, 64, 0, ctypes.byref(c), 0, FAKE, need, None) == MISMATCH
    assert L.fvattn_attn_plan(None, 1, 2, 1024, 64, 0, ctypes.byref(c), 0, FAKE, need, None) == INVALID
    o = fv._OptsC(0, 0, None, 0, -1, 0)
    assert L.fvattn_attn_run(None, FAKE, FAKE, FAKE, 1, 2, 1024, 64, 0, ctypes.byref(c), ctypes.byref(o), FAKE,
                             need, None) == INVALID
    assert L.fvattn_attn_run(FAKE, FAKE, FAKE, FAKE, 1, 2, 1024, 64, 0, ctypes.byref(c), ctypes.byref(o), FAKE,
                             need - 1, None) == WORKSPACE
    o.grid = -1
    assert L.fvattn_attn_run(FAKE, FAKE, FAKE, FAKE, 1, 2, 1024, 64, 0, ctypes.byref(c), ctypes.byref(o), FAKE,
                             need, None) == INVALID


def test_worklist_and_pool_validation(L):
    c = _csr()
    need = L.fvattn_worklist_ws_bytes(2 * 16)
    assert need >= 256 + 2 * 4 * 32 and L.fvattn_worklist_ws_bytes(0) == 0
    assert L.fvattn_worklist(ctypes.byref(c), 7, 1, FAKE, FAKE, need, None) == INVALID
    assert L.fvattn_worklist(None, 0, 1, FAKE, FAKE, need, None) == INVALID
    assert L.fvattn_worklist(ctypes.byref(c), 0, 1, None, FAKE, need, None) == INVALID
    assert L.fvattn_worklist(ctypes.byref(c), 0, 1, FAKE, None, need, None) == INVALID
    assert L.fvattn_worklist(ctypes.byref(c), 0, 3, FAKE, FAKE, need, None) == INVALID      # G not in {1, 2, 4}
    assert L.fvattn_worklist(ctypes.byref(c), 4, 2, FAKE, FAKE, need - 1, None) == WORKSPACE
    big = _csr(5000, 1024)
    assert L.fvattn_worklist(ctypes.byref(big), 4, 1, FAKE, FAKE, 1 << 40, None) == UNSUPPORTED  # > 4096 heads
    st = ctypes.c_uint32(0)
    assert L.fvattn_ws_status(None, 0, ctypes.byref(st), None) == INVALID
    assert L.fvattn_ws_status(FAKE, 2, ctypes.byref(st), None) == INVALID
    assert L.fvattn_ws_status(FAKE, 0, None, None) == INVALID
    assert L.fvattn_pool(FAKE, 2, 1024, 64, 0, 48, FAKE, None) == UNSUPPORTED
    assert L.fvattn_pool(None, 2, 1024, 64, 0, 64, FAKE, None) == INVALID
    assert L.fvattn_pool(FAKE, 2, 0, 64, 0, 64, FAKE, None) == INVALID
    assert L.fvattn_pool(FAKE, 2, 1024, 80, 0, 64, FAKE, None) == UNSUPPORTED


def test_binding_has_no_cpu_path():
    import torch
    x = torch.zeros(1, 1, 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fv.route(x, x, 64, 64, 0.9)
    with pytest.raises(TypeError):
        fv._dtype_code(torch.zeros(1, dtype=torch.float16))


def test_product_never_touches_oracle():
    pkg = os.path.join(ROOT, "top_block_sparse_pooled_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", src), f"{f} mentions the oracle"


def _route_ex(L, opts, B=1, H=2, N=1024, d=64, dt=0, bq=64, bk=64, ws=FAKE, ws_bytes=1 << 40):
    c = _csr(B * H, N, bq, bk)
    return L.fvattn_route_ex(FAKE, FAKE, B, H, N, d, dt, bq, bk,
                             ctypes.byref(opts) if opts is not None else None, ctypes.byref(c), ws, ws_bytes, None)


def _ropts(mode=0, topk=0, p=0.9, k_min=1, k_max=0, window=0):
    return fv._RouteOptsC(mode, topk, p, k_min, k_max, window, 0)


@pytest.mark.parametrize("kw", [
    dict(mode=2), dict(mode=-1), dict(p=0.0), dict(p=1.5), dict(p=math.nan), dict(k_min=0),
    dict(k_min=5, k_max=3), dict(k_max=-1), dict(mode=1, topk=0), dict(mode=1, topk=-3),
    dict(window=-1), dict(mode=1, topk=4, window=-2),
])
def test_route_ex_rejects_bad_options(L, kw):
    assert _route_ex(L, _ropts(**kw)) == INVALID


def test_route_ex_validation_order(L):
    assert _route_ex(L, None) == INVALID
    assert _route_ex(L, _ropts(), d=96) == UNSUPPORTED           # shape checks as fvattn_route
    assert _route_ex(L, _ropts(mode=1, topk=3), dt=5) == UNSUPPORTED
    assert _route_ex(L, _ropts(mode=1, topk=3), ws_bytes=16) == WORKSPACE


def _sopts(groups=2, critical=0, alpha=0.5, tau=0.0):
    return fv._SasaOptsC(groups, critical, alpha, tau, None)


def _route_sasa(L, so, ro=None, B=1, H=2, N=1024, d=64, bq=64, bk=64, ws_bytes=1 << 40):
    c = _csr(B * H, N, bq, bk)
    ro = ro if ro is not None else _ropts()
    return L.fvattn_route_sasa(FAKE, FAKE, B, H, N, d, 0, bq, bk, ctypes.byref(ro),
                               ctypes.byref(so) if so is not None else None, ctypes.byref(c), FAKE, ws_bytes, None)


@pytest.mark.parametrize("kw", [dict(groups=0), dict(groups=3), dict(alpha=-0.1), dict(alpha=1.5),
                                dict(alpha=math.nan), dict(tau=-1.0), dict(tau=2.0), dict(critical=-5)])
def test_route_sasa_rejects_bad_options(L, kw):
    assert _route_sasa(L, _sopts(**kw)) == INVALID     # groups=3 > B*H=2


def test_route_sasa_validation_order(L):
    assert _route_sasa(L, None) == INVALID
    assert _route_sasa(L, _sopts(), ro=_ropts(p=2.0)) == INVALID
    assert _route_sasa(L, _sopts(), d=96) == UNSUPPORTED
    need = L.fvattn_route_sasa_ws_bytes(1, 2, 1024, 64, 64, 64, 2)
    assert need > L.fvattn_route_ws_bytes(1, 2, 1024, 64, 64, 64) + 2 * 16 * 16 * 8
    assert L.fvattn_route_sasa_ws_bytes(1, 2, 1024, 64, 64, 64, 3) == 0
    assert _route_sasa(L, _sopts(), ws_bytes=need - 1) == WORKSPACE


def test_noalloc_validation(L):
    """The no-allocation entry point validates like fvattn_sparse_attn and refuses problems larger
    than its static scratch, all before touching the device."""
    def call(B=1, H=2, N=1024, d=64, dt=0, csr=None, opts=None, v=FAKE):
        c = csr if csr is not None else _csr(B * H, N)
        return L.fvattn_sparse_attn_noalloc(FAKE, FAKE, v, FAKE, B, H, N, d, dt, ctypes.byref(c),
                                            ctypes.byref(opts) if opts is not None else None, None)
    assert call(dt=3) == UNSUPPORTED
    assert call(v=None) == INVALID
    assert call(N=1000, csr=_csr(2, 1024)) == MISMATCH
    assert call(opts=fv._OptsC(9, 0, None, 0, -1, 0)) == INVALID
    assert call(opts=fv._OptsC(0, 0, FAKE, 4 * 16 - 1, -1, 0)) == INVALID      # trace too small
    assert L.fvattn_sparse_attn_noalloc(FAKE, FAKE, FAKE, FAKE, 1, 2, 1024, 64, 0, None, None, None) == INVALID
    # 300 heads x 1280 query blocks = 384,000 rows > FVATTN_NOALLOC_MAX_ROWS (262,144)
    assert call(H=300, N=81920, csr=_csr(300, 81920)) == SCRATCH
    assert call(H=300, N=81920, csr=_csr(300, 81920), dt=7) == UNSUPPORTED   # argument checks come first
