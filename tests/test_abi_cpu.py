"""Host-side checks of the C ABI: the shared library loads, exports every
entry point include/gptq.h declares, and rejects bad arguments before it
touches the GPU (no compute call runs here)."""

import ctypes
import os
import re

import pytest

import post_weight_quantization_15_amd as gq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gptq.h")

FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def header_functions():
    src = open(HEADER, encoding="utf-8").read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gptq_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gq.lib_path()):
        pytest.fail("libgptq_hip.so not built; run __graft_entry__.build()")
    return gq.load_library()


def test_exports_match_header(lib):
    declared = header_functions()
    assert declared == sorted(gq.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    assert lib.gptq_status_string(0) == b"ok"
    assert b"positive definite" in lib.gptq_status_string(2)
    assert lib.gptq_status_string(99) == b"unknown status"


def params(bits=4, g=-1, b=128, damp=0.01, act=0, grid=0, static=0,
           fs=None, fz=None):
    return gq._Params(bits, g, b, damp, act, grid, static, fs, fz)


@pytest.mark.parametrize("kw", [
    dict(bits=5), dict(bits=1), dict(g=0), dict(g=-2), dict(b=0),
    dict(damp=-0.1), dict(damp=float("nan")), dict(damp=float("inf")),
    dict(act=2), dict(g=96, b=128), dict(grid=3), dict(grid=-1), dict(static=2),
    dict(grid=2), dict(grid=2, fs=0x1000), dict(grid=0, fs=0x1000, fz=0x1000),
    dict(grid=1, fz=0x1000),
])
def test_workspace_query_rejects_bad_params(lib, kw):
    p = params(**kw)
    assert lib.gptq_workspace_bytes(256, 512, ctypes.byref(p), 1) == 0


def test_workspace_query_accepts_variants(lib):
    ok = [params(4, 96, 128, static=1), params(2, 8, 128, grid=1),
          params(3, 96, 128, grid=2, fs=0x1000, fz=0x1000),
          params(4, -1, 128, grid=2, fs=0x1000, fz=0x1000), params(8, -1, 7, grid=1)]
    for p in ok:
        assert lib.gptq_workspace_bytes(256, 512, ctypes.byref(p), 1) > 0


def test_workspace_query_sizes(lib):
    p = params(4, 128, 128)
    inside = lib.gptq_workspace_bytes(4096, 4096, ctypes.byref(p), 1)
    outside = lib.gptq_workspace_bytes(4096, 4096, ctypes.byref(p), 0)
    assert inside > outside > 4096 * 4096 * 4
    assert lib.gptq_workspace_bytes(0, 4096, ctypes.byref(p), 1) == 0
    assert lib.gptq_hessian_workspace_bytes(-1, 10) == 0
    assert lib.gptq_factor_workspace_bytes(0) == 0
    assert lib.gptq_factor_workspace_bytes(4096) >= 2 * 4096 * 4096 * 8


def test_hessian_rejects(lib):
    INV = gq.GPTQ_ERR_INVALID_ARG
    assert lib.gptq_hessian_accumulate(None, 16, FAKE, 0, 4, 16, None, 0, None) == INV
    assert lib.gptq_hessian_accumulate(FAKE, 0, FAKE, 0, 4, 16, None, 0, None) == INV
    assert lib.gptq_hessian_accumulate(FAKE, 16, FAKE, 0, -1, 16, None, 0, None) == INV
    assert lib.gptq_hessian_accumulate(FAKE, 16, FAKE, 0, 4, 8, None, 0, None) == INV
    assert lib.gptq_hessian_accumulate(FAKE, 16, FAKE, 7, 4, 16, None, 0, None) == INV
    assert lib.gptq_hessian_accumulate(FAKE, 16, None, 0, 4, 16, None, 0, None) == INV
    assert lib.gptq_hessian_accumulate(FAKE, 70000, FAKE, 0, 4, 70000, None, 0, None) == INV
    need = lib.gptq_hessian_workspace_bytes(4096, 262144)
    assert need > 0
    assert lib.gptq_hessian_accumulate(FAKE, 4096, FAKE, 0, 262144, 4096, FAKE,
                                       need - 1, None) == gq.GPTQ_ERR_WORKSPACE


def test_cholesky_inverse_rejects(lib):
    INV = gq.GPTQ_ERR_INVALID_ARG
    f = ctypes.c_float(0)
    args = [FAKE, 10, 16, 0.01, 0, FAKE, FAKE, FAKE, ctypes.byref(f), FAKE, 1 << 30, None]
    for idx, bad in [(0, None), (1, 0), (2, 0), (3, -1.0), (3, float("nan")),
                     (4, 3), (5, None), (6, None), (7, None)]:
        a = list(args)
        a[idx] = bad
        assert lib.gptq_cholesky_inverse(*a) == INV, idx
    a = list(args)
    a[10] = 16
    assert lib.gptq_cholesky_inverse(*a) == gq.GPTQ_ERR_WORKSPACE


def quant_args(p, **over):
    a = dict(W=FAKE, dt=0, m=16, d=32, ldw=32, S=FAKE, n=10, p=ctypes.byref(p),
             R=None, perm=None, dead=None, qw=FAKE, sc=FAKE, zr=FAKE, gi=FAKE,
             wh=None, ws=FAKE, wsb=1 << 40, st=None)
    a.update(over)
    return list(a.values())


def test_quantize_layer_rejects(lib):
    INV = gq.GPTQ_ERR_INVALID_ARG
    p = params()
    q = lib.gptq_quantize_layer
    assert q(*quant_args(p, W=None)) == INV
    assert q(*quant_args(p, m=0)) == INV
    assert q(*quant_args(p, ldw=16)) == INV
    assert q(*quant_args(p, dt=3)) == INV
    assert q(*quant_args(p, qw=None)) == INV
    assert q(*quant_args(p, sc=None)) == INV
    assert q(*quant_args(p, zr=None)) == INV
    assert q(*quant_args(p, gi=None)) == INV
    assert q(*quant_args(p, R=FAKE)) == INV                 # R without perm/dead
    assert q(*quant_args(p, S=None)) == INV                 # factoring needs S
    assert q(*quant_args(p, n=0)) == INV
    bad = params(bits=7)
    assert q(*quant_args(bad)) == INV
    bad = params(g=24, b=32)                                # group straddles blocks
    assert q(*quant_args(bad, d=64)) == INV
    assert q(*quant_args(p, wsb=100)) == gq.GPTQ_ERR_WORKSPACE
    assert q(*quant_args(p, ws=None)) == gq.GPTQ_ERR_WORKSPACE


def test_binding_refuses_host_tensors():
    import torch
    S = torch.zeros(4, 4)
    X = torch.zeros(3, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gq.gptq_hessian_accumulate(S, X)


def test_noalloc_hessian_rejects(lib):
    INV = gq.GPTQ_ERR_INVALID_ARG
    f = lib.gptq_hessian_accumulate_noalloc
    assert f(None, 16, FAKE, 0, 4, 16, None) == INV
    assert f(FAKE, 0, FAKE, 0, 4, 16, None) == INV
    assert f(FAKE, 16, FAKE, 0, -1, 16, None) == INV
    assert f(FAKE, 16, FAKE, 0, 4, 8, None) == INV
    assert f(FAKE, 16, FAKE, 7, 4, 16, None) == INV
    assert f(FAKE, 16, None, 0, 4, 16, None) == INV
    assert f(FAKE, 70000, FAKE, 0, 4, 70000, None) == INV


def test_binding_rejects_overlapping_rows_and_wrong_types():
    """Checks done before any device pointer is taken (CPU tensors)."""
    import torch
    S = torch.zeros(8, 8)
    X = torch.zeros(1, 8).expand(5, 8)          # stride (0, 1): rows overlap
    with pytest.raises(ValueError, match="overlap"):
        gq.gptq_hessian_accumulate(S, X)
    with pytest.raises(ValueError, match="overlap"):
        gq.gptq_hessian_accumulate_noalloc(S, X)
    with pytest.raises(TypeError):
        gq.gptq_hessian_accumulate(S.double(), torch.zeros(5, 8))
    W = torch.zeros(1, 8).expand(4, 8)
    with pytest.raises(ValueError, match="overlap"):
        gq.gptq_quantize_layer(W, S, 5)
    W = torch.zeros(4, 8)
    with pytest.raises(TypeError, match="perm"):
        gq.gptq_quantize_layer(W, None, 0, R=torch.zeros(8, 8),
                               perm=torch.zeros(8, dtype=torch.int64),
                               dead=torch.zeros(8, dtype=torch.uint8))
    with pytest.raises(TypeError, match="R"):
        gq.gptq_quantize_layer(W, None, 0, R=torch.zeros(8, 8, dtype=torch.float64),
                               perm=torch.zeros(8, dtype=torch.int32),
                               dead=torch.zeros(8, dtype=torch.uint8))
    with pytest.raises(ValueError, match="together"):
        gq.gptq_quantize_layer(W, S, 5, R=torch.zeros(8, 8))
    with pytest.raises(ValueError):
        gq.gptq_cholesky_inverse(torch.zeros(8, 7), 5)
    with pytest.raises(ValueError, match="contiguous"):
        gq.gptq_cholesky_inverse(torch.zeros(8, 8).T, 5)
    with pytest.raises(TypeError):
        gq.gptq_cholesky_inverse(torch.zeros(8, 8, dtype=torch.float64), 5)


def test_dequant_matmul_rejects(lib):
    INV = gq.GPTQ_ERR_INVALID_ARG
    f = lib.gptq_dequant_matmul
    ok = dict(X=FAKE, dt=0, n=4, d=64, ldx=64, qw=FAKE, sc=FAKE, sdt=1, zp=FAKE, gi=FAKE,
              m=32, bits=4, g=32, sgn=0, Y=FAKE, ldy=32)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["X"], a["dt"], a["n"], a["d"], a["ldx"], a["qw"], a["sc"], a["sdt"],
                 a["zp"], a["gi"], a["m"], a["bits"], a["g"], a["sgn"], a["Y"], a["ldy"], None)

    for kw in (dict(dt=1), dict(dt=2), dict(sdt=0), dict(sdt=3), dict(n=-1), dict(d=0),
               dict(m=0), dict(ldx=63), dict(ldy=31),
               dict(bits=5), dict(g=0), dict(g=-2), dict(sgn=2), dict(X=None),
               dict(qw=None), dict(sc=None), dict(zp=None), dict(gi=None), dict(Y=None),
               dict(d=70000, ldx=70000)):
        assert call(**kw) == INV, kw
    # n = 0 launches nothing and succeeds without a GPU (fp32 or fp16 scales)
    assert call(n=0, X=None, Y=None) == gq.GPTQ_OK
    assert call(n=0, X=None, Y=None, sdt=2) == gq.GPTQ_OK


def test_stack_rejects(lib):
    """Descriptor validation of the layer-by-layer driver (no GPU work)."""
    INV = gq.GPTQ_ERR_INVALID_ARG
    F = 0x1000

    def layer(m, d, **kw):
        p = params(**kw)
        return gq._StackLayer(F, 0, m, d, d, p, F, F, F, F)

    two = (gq._StackLayer * 2)(layer(64, 128), layer(32, 64))
    assert lib.gptq_stack_workspace_bytes(two, 2, 1000) > 0
    bad_dims = (gq._StackLayer * 2)(layer(64, 128), layer(32, 65))
    assert lib.gptq_quantize_stack(bad_dims, 2, FAKE, 1000, 0, FAKE, None, FAKE,
                                   1 << 40, None) == INV
    assert lib.gptq_quantize_stack(two, 2, FAKE, 1000, 3, FAKE, None, FAKE, 1 << 40,
                                   None) == INV
    assert lib.gptq_quantize_stack(two, 2, None, 1000, 0, FAKE, None, FAKE, 1 << 40,
                                   None) == INV
    assert lib.gptq_quantize_stack(two, 2, FAKE, 0, 0, FAKE, None, FAKE, 1 << 40,
                                   None) == INV
    assert lib.gptq_quantize_stack(two, 0, FAKE, 10, 0, FAKE, None, FAKE, 1 << 40,
                                   None) == INV
    badp = (gq._StackLayer * 1)(layer(64, 128, bits=5))
    assert lib.gptq_stack_workspace_bytes(badp, 1, 1000) == 0
    assert lib.gptq_quantize_stack(two, 2, FAKE, 1000, 0, FAKE, None, FAKE, 16,
                                   None) == gq.GPTQ_ERR_WORKSPACE


def test_trace_host_side(lib):
    """Tracing state is host-side: enabling, reading with nothing recorded
    and rejecting bad arguments need no GPU."""
    import ctypes as C
    ms = (C.c_double * 5)()
    n = (C.c_int64 * 5)()
    assert lib.gptq_trace_enable(2) == gq.GPTQ_ERR_INVALID_ARG
    assert lib.gptq_trace_read(None, None, 0) == gq.GPTQ_ERR_INVALID_ARG
    assert lib.gptq_trace_read(ms, n, 1) == gq.GPTQ_OK
    assert lib.gptq_trace_read(ms, n, 0) == gq.GPTQ_OK and list(n) == [0] * 5
    assert lib.gptq_trace_enable(1) == gq.GPTQ_OK
    assert lib.gptq_trace_enable(0) == gq.GPTQ_OK
