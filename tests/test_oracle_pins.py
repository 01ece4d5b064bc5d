"""Pins of the float64 oracle to the numbers the pages print.

Each case reads a fixture under tests/golden/ whose "source" field names the
page and section the values come from.  None of these values were produced by
the code under test.
"""

import numpy as np
import pytest

import oracle as orc
from conftest import load_golden


def test_toy_obs_example():
    """[teardown] toy example: H = 2XX^T, diag H^-1, greedy criterion,
    compensation of w2 and the output distance before/after."""
    g = load_golden("toy_obs.json")
    tol = g["printed_digits_abs_tol"]
    w = np.array(g["w"])
    X = np.array(g["X"])
    H = 2.0 * X @ X.T                  # the toy uses H = 2 X X^T
    np.testing.assert_allclose(H, g["H"], atol=1e-12)
    Hinv = np.linalg.inv(H)
    np.testing.assert_allclose(np.diag(Hinv), g["hinv_diag"], atol=tol)
    grid = np.array(g["grid"])
    quant = grid[np.argmin(np.abs(w[:, None] - grid[None, :]), axis=1)]
    np.testing.assert_allclose(quant, g["quant_w"])
    crit = orc.obs_criterion(w, quant, H)
    np.testing.assert_allclose(crit, g["criterion"], atol=tol)
    assert int(np.argmin(crit)) == g["first_quantized"]
    # quantize w1 and compensate w2 with the OBS update (eq. (22))
    p = g["first_quantized"]
    delta, _ = orc.obs_update(Hinv, p, w[p] - quant[p])
    w_new = w + delta
    assert abs(w_new[p] - quant[p]) < 1e-12
    assert abs(w_new[1] - g["w2_after_compensation"]) < tol
    w_unc = w.copy()
    w_unc[p] = quant[p]
    dist_unc = np.linalg.norm(w @ X - w_unc @ X)
    dist_comp = np.linalg.norm(w @ X - w_new @ X)
    assert abs(dist_unc - g["output_distance_uncompensated"]) < tol
    assert abs(dist_comp - g["output_distance_compensated"]) < tol
    assert dist_comp < dist_unc


def test_encode_example():
    """[derivation] 1.1: Delta=0.25, z=8, w=0.62 -> 2.48 -> c=10 -> q=0.50."""
    g = load_golden("encode_example.json")
    c, q, v = orc.encode(np.array([g["w"]]), np.array([g["scale"]]),
                         np.array([g["zero"]]), g["bits"])
    assert abs(v[0] - g["v"]) < 1e-12
    assert int(c[0]) == g["code"]
    assert abs(q[0] - g["q"]) < 1e-12


def test_two_d_compensation_and_R_form():
    """[derivation] 4.1 / 9.2: delta = [-0.12, +0.06]; the same step through
    the upper Cholesky factor R of G; next conditional inverse R_11^2."""
    g = load_golden("two_d_compensation.json")
    G = np.array(g["G"])
    w = np.array(g["w_work"])
    delta, _ = orc.obs_update(G, g["p"], g["rho"])
    np.testing.assert_allclose(delta, g["delta"], atol=1e-12)
    np.testing.assert_allclose(w + delta, g["w_new"], atol=1e-12)
    # the oracle's factor route applied to H = G^-1 with no damping
    R, _ = orc.factor(np.linalg.inv(G), 0.0)
    np.testing.assert_allclose(R, g["R"], atol=1e-12)
    eta = g["rho"] / R[0, 0]
    np.testing.assert_allclose(w - eta * R[0, :], g["w_new"], atol=1e-12)
    assert abs(R[1, 1] ** 2 - g["next_conditional_inverse"]) < 1e-12


def test_downdate_counterexample():
    """[derivation] section 6: freezing a coordinate needs the rank-1
    downdate (1/2), not a truncation of the old inverse (2/3)."""
    g = load_golden("downdate_counterexample.json")
    H = np.array(g["H_F"])
    G = np.linalg.inv(H)
    Gt = orc.downdate(G, g["p"])
    assert abs(Gt[0, 0] - g["G_T"]) < 1e-12
    assert abs(G[1, 1] - g["plain_truncation_wrong"]) < 1e-12


def test_multi_constraint_example():
    """[derivation] 7.2 / 7.3: delta*, cost, Gamma, Gamma^-1 and G_T."""
    g = load_golden("multi_constraint_3d.json")
    H = np.array(g["H_F"])
    G = np.linalg.inv(H)
    np.testing.assert_allclose(4.0 * G, g["G_F_times_4"], atol=1e-12)
    out = orc.block_update(G, g["B"], g["a_B"])
    np.testing.assert_allclose(out["Gamma"], g["Gamma"], atol=1e-12)
    np.testing.assert_allclose(np.linalg.inv(out["Gamma"]), g["Gamma_inv"],
                               atol=1e-12)
    np.testing.assert_allclose(out["delta"], g["delta"], atol=1e-12)
    assert abs(out["cost"] - g["cost"]) < 1e-12
    np.testing.assert_allclose(out["G_T"], [[g["G_T"]]], atol=1e-12)
    # freezing the middle coordinate instead costs 2 (the page's comparison)
    frozen = np.array([-1.0, 0.0, -1.0])
    assert abs(0.5 * frozen @ H @ frozen - g["cost_if_middle_frozen"]) < 1e-12


def test_sixteen_level_example_full_loop():
    """[derivation] section 11: the whole layer through the oracle's main
    loop with the page's fixed grid and lambda = 0."""
    g = load_golden("sixteen_level_example.json")
    A0 = np.array(g["A0"])
    X = A0.T                                   # eq. (5): X = reshape(A)^T
    np.testing.assert_allclose(X, g["X"])
    W = np.array(g["W"])
    N = X.shape[1]
    np.testing.assert_allclose(W @ X, g["Y"], atol=1e-12)
    S = orc.hessian_sum(A0)                    # token-major input
    np.testing.assert_allclose(S, g["XXt"], atol=1e-12)
    np.testing.assert_allclose(orc.hessian_from_sum(S, N), g["H"], atol=1e-12)
    m = W.shape[0]
    grid = (np.full(m, g["scale"], dtype=np.float32),
            np.full(m, g["zero"], dtype=np.int64))
    res = orc.gptq_layer(W, S, N, bits=g["bits"], group_size=-1,
                         blocksize=128, percdamp=0.0, act_order=False,
                         damp_override=0.0, fixed_grid=grid)
    np.testing.assert_allclose(res.R.T @ res.R, g["G"], atol=1e-12)
    np.testing.assert_array_equal(res.codes, g["K"])
    np.testing.assert_allclose(res.w_hat, g["W_hat"], atol=1e-12)
    np.testing.assert_allclose(res.rho_perm[:, 0], g["rho0"], atol=1e-12)
    np.testing.assert_allclose(res.rho_perm[:, 1], g["rho1"], atol=1e-12)
    tol = g["printed_digits_abs_tol"]
    dl = res.rho_perm ** 2 / (2.0 * np.diag(res.R)[None, :] ** 2)
    np.testing.assert_allclose(dl[:, 0], g["dl0"], atol=tol)
    np.testing.assert_allclose(dl[:, 1], g["dl1"], atol=tol)
    np.testing.assert_allclose((res.w_hat - W) @ X, g["Yhat_minus_Y"],
                               atol=1e-12)
    err = orc.layer_error(W, res.w_hat, S, N)
    assert abs(err * N - g["sum_sq_err"]) < 1e-12
    assert abs(err - g["layer_error"]) < tol
    # eq. (67): layer error = sum of the per-step increments over both rows
    assert abs(err - orc.proxy_loss(res.rho_perm, res.R)) < 1e-12
    # eq. (68): RTN under the same grid
    _, q_rtn = orc.rtn(W, grid[0], grid[1], g["bits"])
    np.testing.assert_allclose(q_rtn, g["W_rtn"], atol=1e-12)
    err_rtn = orc.layer_error(W, q_rtn, S, N)
    assert abs(err_rtn - g["rtn_layer_error"]) < 1e-12
    assert abs(err / err_rtn - g["ratio_gptq_over_rtn"]) < 5e-5
    # the intermediate working matrix after column 0 (eq. (59)) via the
    # per-block loop with blocksize 1 (the tail update is then the lazy GEMM)
    res1 = orc.quantize_columns(W, res.R, 4, -1, 1, grid)
    np.testing.assert_allclose(res1["q"], g["W_hat"], atol=1e-12)


def test_damping_example():
    """[derivation] eq. (12) and the section 10 damping and dead-feature
    lines on a hand-worked case: a never-seen feature gets the placeholder
    diagonal 1 BEFORE the mean is taken; lambda = percdamp * mean(diag H)."""
    g = load_golden("damping_example.json")
    tok = np.array(g["tokens"])
    S = orc.hessian_sum(tok)
    n = tok.shape[0]
    for act in (False, True):
        H, perm, dead, damp = orc.prepare(S, n, g["percdamp"], act)
        np.testing.assert_array_equal(dead, g["dead"])
        assert abs(damp - g["damp"]) < 1e-15
        np.testing.assert_allclose(np.diag(H)[np.argsort(perm)],
                                   g["diag_after_dead_fix"], atol=1e-15)
        if act:
            np.testing.assert_array_equal(perm, g["perm_act_order"])
            np.testing.assert_allclose(H, g["H_perm_act_order"], atol=1e-15)
    # the damped matrix the factor inverts: R^T R (H + lambda I) = I
    H, perm, dead, damp = orc.prepare(S, n, g["percdamp"], True)
    R, used = orc.factor(H, damp)
    assert used == damp
    np.testing.assert_allclose(R.T @ R @ (np.array(g["H_perm_act_order"]) +
                                          g["damp"] * np.eye(3)), np.eye(3),
                               atol=1e-12)
    c2 = g["second_case"]
    _, _, _, damp2 = orc.prepare(np.diag(c2["S_diag"]), c2["n"], 0.01, False)
    assert abs(damp2 - c2["damp"]) < 1e-15


def test_zero_point_rounds_to_nearest():
    """[derivation] 1.1: z = clip(round(-w_min / Delta), 0, 15).  The row
    [-1.15, 1.85] has Delta = 3/15 = 0.2 and -w_min / Delta = 5.75, whose
    nearest integer is 6 (flooring would give 5)."""
    sc, z = orc.fit_grid(np.array([[-1.15, 1.85, 0.3]]), 4)
    assert abs(float(sc[0]) - 0.2) < 1e-7
    assert int(z[0]) == 6
    # 0 is represented exactly and the extremes land within half a step
    c, q, _ = orc.encode(np.array([0.0, -1.15, 1.85]), sc[0], z[0], 4)
    assert q[0] == 0.0
    assert abs(q[1] + 1.15) <= 0.1 + 1e-7 and abs(q[2] - 1.85) <= 0.1 + 1e-7


def test_sixteen_level_example_dequant_matmul():
    """[derivation] section 11: the stored codes K with Delta = 0.25, z = 8
    dequantize to the page's W_hat, and the quantized layer's outputs are
    the page's Y plus its printed Y_hat - Y."""
    g = load_golden("sixteen_level_example.json")
    K = np.array(g["K"])
    packed = orc.pack_codes(K, 4)
    sc = np.full((2, 1), g["scale"])
    z = np.full((2, 1), g["zero"])
    gi = np.zeros(2, dtype=np.int64)
    np.testing.assert_allclose(orc.dequantize(packed, sc, z, gi, 2, 4), g["W_hat"],
                               atol=1e-15)
    Y_hat = orc.dequant_matmul(np.array(g["A0"]), packed, sc, z, gi, 4)
    np.testing.assert_allclose(Y_hat.T, np.array(g["Y"]) + np.array(g["Yhat_minus_Y"]),
                               atol=1e-12)
