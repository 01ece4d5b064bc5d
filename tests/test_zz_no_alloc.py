"""The allocation-free Hessian entry point against the workspace one,
through the C ABI: two calls in a row on one GPU, the second smaller, each
compared with gptq_hessian_accumulate on the same input.

Where both entry points plan the same token split the results are the same
bits; where the scratch size forces fewer splits (the attention-projection
workload) they differ only by fp32 summation rounding, bounded entrywise by
the longer chain: |dS_ij| <= 2 * (steps per split) * 2^-24 * sqrt(S_ii S_jj)
(each side's error is at most steps * 2^-24 * sum_t |x_ti x_tj|, Cauchy-
Schwarz); both are also held to exact float64 sums on sampled features.
"""

import ctypes
import math

import numpy as np
import pytest
import torch

import oracle as orc
import post_weight_quantization_15_amd as gq
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return gq.load_library()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _both(lib, X):
    dev = X.device
    n, d = X.shape
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    S_ws = torch.zeros(d, d, dtype=torch.float32, device=dev)
    need = lib.gptq_hessian_workspace_bytes(d, n)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    rc = lib.gptq_hessian_accumulate(_ptr(S_ws), d, _ptr(X), gq.GPTQ_BF16, n, d,
                                     _ptr(ws), ws.numel(), st)
    assert rc == gq.GPTQ_OK
    S_na = torch.zeros(d, d, dtype=torch.float32, device=dev)
    rc = lib.gptq_hessian_accumulate_noalloc(_ptr(S_na), d, _ptr(X), gq.GPTQ_BF16,
                                             n, d, st)
    assert rc == gq.GPTQ_OK
    torch.cuda.synchronize()
    return S_ws, S_na, need


def _check_pair(S_ws, S_na, X, exact, rng):
    d = X.shape[1]
    n = X.shape[0]
    assert bool(torch.equal(S_na, S_na.t()))
    if exact:
        assert bool(torch.equal(S_ws, S_na))
        return
    diag = torch.diagonal(S_ws).double()
    scale = torch.sqrt(diag[:, None] * diag[None, :]) + 1e-30
    err = float(((S_ws.double() - S_na.double()).abs() / scale).max())
    bound = 2 * math.ceil(n / 32) * 2.0 ** -24
    assert err <= bound, (err, bound)
    cols = np.sort(rng.choice(d, size=32, replace=False))
    idx = torch.from_numpy(cols).to(X.device)
    So = orc.hessian_sum(X.index_select(1, idx).cpu().to(torch.float64).numpy())
    for S in (S_ws, S_na):
        Sg = S.index_select(0, idx).index_select(1, idx).cpu().double().numpy()
        assert np.linalg.norm(Sg - So) / np.linalg.norm(So) <= 1e-5


def test_noalloc_matches_workspace_entry(lib):
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(5)
    # first call: the benchmarked attention-projection input (4096 features,
    # 262144 tokens); the scratch bound gives it fewer token splits
    L = synth.attn_proj_layer(dev)
    X = L["X"]
    S_ws, S_na, need = _both(lib, X)
    print(f"d=4096 n=262144: workspace entry needs {need} B, scratch "
          f"{gq.GPTQ_NOALLOC_SCRATCH_BYTES} B", flush=True)
    _check_pair(S_ws, S_na, X, exact=need <= gq.GPTQ_NOALLOC_SCRATCH_BYTES, rng=rng)
    del L, X, S_ws, S_na
    torch.cuda.empty_cache()
    # second call, smaller (ragged d, 3000 tokens): the same split plan, the
    # same bits; the scratch still holds the first call's partials
    X2 = synth.attn_proj_layer("cpu", m=8, d=648, n=3000)["X"].to(dev)
    S_ws2, S_na2, need2 = _both(lib, X2)
    assert need2 <= gq.GPTQ_NOALLOC_SCRATCH_BYTES
    _check_pair(S_ws2, S_na2, X2, exact=True, rng=rng)
    # accumulating a second chunk onto the first gives the same sum as the
    # workspace entry point doing the same
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    rc = lib.gptq_hessian_accumulate_noalloc(_ptr(S_na2), 648, _ptr(X2), gq.GPTQ_BF16,
                                             3000, 648, st)
    assert rc == gq.GPTQ_OK
    ws = torch.empty(max(need2, 1), dtype=torch.uint8, device=dev)
    rc = lib.gptq_hessian_accumulate(_ptr(S_ws2), 648, _ptr(X2), gq.GPTQ_BF16, 3000,
                                     648, _ptr(ws), ws.numel(), st)
    assert rc == gq.GPTQ_OK
    torch.cuda.synchronize()
    assert bool(torch.equal(S_ws2, S_na2))
