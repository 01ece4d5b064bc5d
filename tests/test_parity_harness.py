"""The GPU-vs-oracle comparison itself, exercised on the CPU with oracle
runs standing in for the GPU: a run on a slightly perturbed Hessian (the
statistics rounded to fp32, as the GPU holds them) takes other valid GPTQ
trajectories after near-ties and must be accepted, with its whole-layer
figures matching the tie-forced oracle; a planted wrong code far from any
rounding boundary must be rejected."""

import numpy as np
import pytest

import oracle as orc
import synth
from parity import compare_layer


def _gpu_like(res, bits):
    return dict(qweight=res.packed.view(np.int32), scales=res.scales,
                zeros=res.zeros.astype(np.uint8), g_idx=res.g_idx.astype(np.int32),
                w_hat=res.w_hat.astype(np.float32))


@pytest.fixture(scope="module")
def layer():
    P = synth.mlp_pair("cpu", d=384, dff=640, n=4096)
    L = P["up"]
    W = L["W"].double().numpy()
    S = orc.hessian_sum(L["X"].double().numpy())
    return W, S, L["X"].shape[0], dict(L["params"])


def test_perturbed_hessian_run_is_accepted(layer):
    W, S, n, params = layer
    res = orc.gptq_layer(W, S, n, **params)
    other = orc.gptq_layer(W, S.astype(np.float32).astype(np.float64), n, **params)
    rep = compare_layer(res, W, S, n, _gpu_like(other, params["bits"]), params)
    assert rep["rows_diverged"] >= 1            # the case exercises divergence
    assert rep["forced"] >= 1 and rep["bad_code"] == 0


def test_planted_wrong_code_is_rejected(layer):
    W, S, n, params = layer
    res = orc.gptq_layer(W, S, n, **params)
    bad = orc.gptq_layer(W, S, n, **params)
    # a code whose pre-rounding value is far from a boundary, moved by one
    j = res.perm[5]
    r = int(np.argmax(np.abs(res.v_perm[:, 5] - np.round(res.v_perm[:, 5])) < 0.2))
    codes = bad.codes.copy()
    codes[r, j] = codes[r, j] + (1 if codes[r, j] < 2 ** params["bits"] - 1 else -1)
    bad.packed = orc.pack_codes(codes, params["bits"])
    with pytest.raises(AssertionError):
        compare_layer(res, W, S, n, _gpu_like(bad, params["bits"]), params)
