"""Comparison of the HIP path's outputs with the float64 oracle.

GPTQ's column chain is chaotic: one code that lands on the other side of a
rounding boundary changes every later code in its row, and both outcomes are
correct.  So the comparison has two parts:

1. Unique results are compared directly with the independent oracle run:
   permutation, dead mask, group index, the packing of the GPU's own codes,
   and -- on rows whose codes all agree -- scales and zero points.  The raw
   element mismatch rate against the oracle is reported.
2. The GPU's whole trajectory is validated by a replay: the oracle's loop is
   re-run in float64 from the same inputs, and at every decision (zero point
   at a group start, code of every weight) the GPU's choice is taken; each
   GPU choice must equal the replay's own or sit within `band` (in units of
   the grid step) of the replay's rounding boundary.  Until a row's first
   mismatch the replay is exactly the independent oracle's state, so first
   divergences are judged against the oracle itself.

The replay uses the oracle's primitives (grid fit, encoder); its state never
serves as an expected value.
"""

from __future__ import annotations

import numpy as np

import oracle as orc

BAND = 1e-3          # near-tie band, in units of the grid step
SCALE_RTOL = 1e-3


def tie_distance(v):
    """Distance of a pre-rounding value to the nearest half-integer."""
    v = np.asarray(v, dtype=np.float64)
    return np.abs(v - np.floor(v) - 0.5)


def replay(Wp, R, bits, group_size, blocksize, codes_perm, scales, zeros,
           row_grid=None, band=BAND):
    """Replay the column loop with the GPU's decisions forced.

    Wp: [m, d] oracle working copy in processing order (dead columns zeroed);
    R: oracle factor; codes_perm: GPU codes in processing order;
    scales/zeros: GPU [m, n_g]; row_grid: GPU (scale, zero) for g = -1.
    Returns a dict of counts.
    """
    W = np.array(Wp, dtype=np.float64, copy=True)
    m, d = W.shape
    maxq = 2 ** bits - 1
    bad_code = bad_zero = bad_scale = forced = 0
    if group_size == -1:
        scale = np.asarray(row_grid[0], dtype=np.float32)
        zero = np.asarray(row_grid[1], dtype=np.int64)
    for i in range(0, d, blocksize):
        i2 = min(i + blocksize, d)
        E = np.zeros((m, i2 - i))
        for j in range(i, i2):
            if group_size > 0 and j % group_size == 0:
                grp = W[:, j:min(j + group_size, d)]
                s_r, z_r = orc.fit_grid(grp, bits)
                lo32 = np.minimum(grp.min(axis=1), 0.0).astype(np.float32)
                zsrc = (-lo32 / s_r).astype(np.float64)
                g = j // group_size
                zg = np.asarray(zeros[:, g], dtype=np.int64)
                sg = np.asarray(scales[:, g], dtype=np.float32)
                zdiff = zg != z_r
                bad_zero += int(np.sum(zdiff & (tie_distance(zsrc) >= band)))
                forced += int(np.sum(zdiff))
                rel = np.abs(sg.astype(np.float64) - s_r) / s_r
                bad_scale += int(np.sum(~zdiff & (rel > SCALE_RTOL)))
                scale, zero = sg, zg
            c_r, _, v = orc.encode(W[:, j], scale, zero, bits)
            cg = np.asarray(codes_perm[:, j], dtype=np.int64)
            cdiff = cg != c_r
            # a boundary only separates codes inside [0, maxq]; the band test
            # on v covers both the rounding and the clipping thresholds
            bad_code += int(np.sum(cdiff & (tie_distance(v) >= band)))
            forced += int(np.sum(cdiff))
            q = scale.astype(np.float64) * (cg - zero)
            eta = (W[:, j] - q) / R[j, j]
            W[:, j:i2] -= eta[:, None] * R[j, j:i2][None, :]
            E[:, j - i] = eta
        W[:, i2:] -= E @ R[i:i2, i2:]
    return dict(bad_code=bad_code, bad_zero=bad_zero, bad_scale=bad_scale,
                forced=forced, maxq=maxq)


def unpack_gpu(qweight, d, bits):
    return orc.unpack_codes(np.asarray(qweight).view(np.uint32), d, bits)


def compare_layer(res, W, S, n, gpu, params, check_w_hat=True):
    """Full comparison of one quantized layer.

    res: oracle GPTQResult from the same inputs; W: original weights (f64
    numpy); S: oracle statistics; gpu: dict of numpy arrays from the HIP path
    (qweight, scales, zeros, g_idx, optionally w_hat).  Returns a report and
    raises AssertionError on any failure.
    """
    bits, g, b = params["bits"], params["group_size"], params["blocksize"]
    m, d = W.shape
    qweight = np.asarray(gpu["qweight"])
    codes_gpu = unpack_gpu(qweight, d, bits)
    # packing is integer work: bit-exact against the oracle's packer
    np.testing.assert_array_equal(orc.pack_codes(codes_gpu, bits),
                                  qweight.view(np.uint32))
    np.testing.assert_array_equal(np.asarray(gpu["g_idx"]), res.g_idx)
    scales = np.asarray(gpu["scales"], dtype=np.float32)
    zeros = np.asarray(gpu["zeros"], dtype=np.int64)
    assert scales.shape == res.scales.shape and zeros.shape == res.zeros.shape
    codes_perm = codes_gpu[:, res.perm]
    mism = codes_perm != res.codes_perm
    rows_div = np.nonzero(mism.any(axis=1))[0]
    clean = np.setdiff1d(np.arange(m), rows_div)
    if g == -1:
        # fitted on the original weights: identical inputs, exact result
        np.testing.assert_array_equal(zeros, res.zeros)
        np.testing.assert_array_equal(scales, res.scales)
    else:
        zmis = zeros[clean] != res.zeros[clean]
        assert not zmis.any(), f"zero points differ on {int(zmis.sum())} clean entries"
        rel = np.abs(scales[clean].astype(np.float64) - res.scales[clean]) / res.scales[clean]
        assert rel.max(initial=0.0) <= SCALE_RTOL, f"scale rel err {rel.max()}"
    Wp = np.array(W, dtype=np.float64)
    Wp[:, res.dead] = 0.0
    Wp = Wp[:, res.perm]
    rg = (scales[:, 0], zeros[:, 0]) if g == -1 else None
    rep = replay(Wp, res.R, bits, g, b, codes_perm, scales, zeros, rg)
    assert rep["bad_code"] == 0 and rep["bad_zero"] == 0 and rep["bad_scale"] == 0, rep
    ng = scales.shape[1]
    gid = res.g_idx if g > 0 else np.zeros(d, dtype=np.int64)
    w_hat_codes = scales[np.arange(m)[:, None], gid[None, :]].astype(np.float64) * \
        (codes_gpu - zeros[np.arange(m)[:, None], gid[None, :]])
    report = dict(mismatch_elems=int(mism.sum()), mismatch_rate=float(mism.mean()),
                  rows_diverged=int(rows_div.size), forced=rep["forced"], n_groups=ng)
    if check_w_hat and "w_hat" in gpu:
        w_hat = np.asarray(gpu["w_hat"], dtype=np.float64)
        np.testing.assert_allclose(w_hat, w_hat_codes, rtol=1e-6, atol=0)
    rel_w = np.linalg.norm(w_hat_codes - res.w_hat) / max(np.linalg.norm(res.w_hat), 1e-30)
    assert rel_w <= 1e-3, f"||dW_hat||/||W_hat|| = {rel_w}"
    L_orc = orc.layer_error(W, res.w_hat, S, n)
    L_gpu = orc.layer_error(W, w_hat_codes, S, n)
    rel_L = abs(L_gpu - L_orc) / max(L_orc, 1e-300)
    assert rel_L <= 1e-3, f"layer error rel diff {rel_L} ({L_gpu} vs {L_orc})"
    report.update(w_hat_rel=float(rel_w), layer_err_rel=float(rel_L),
                  layer_err=float(L_orc))
    return report
