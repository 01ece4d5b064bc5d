"""Comparison of the HIP path's outputs with the float64 oracle.

GPTQ's column chain is chaotic: one code that lands on the other side of a
rounding boundary changes every later code in its row, and both outcomes are
correct.  So the comparison has two parts:

1. Unique results are compared directly with the independent oracle run:
   permutation, dead mask, group index, the packing of the GPU's own codes,
   and -- on each row's prefix before its first divergence (a code or a
   zero point that landed on the other side of a near-tie) -- the codes,
   scales, zero points and dequantized weights.  The raw element mismatch
   rate, the number of diverged rows and the unique fraction are reported;
   the layer error is compared over the whole layer.
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


def compare_layer(res, W, S, n, gpu, params, check_w_hat=True, sampled_rows=False):
    """Full comparison of one quantized layer.

    res: oracle GPTQResult from the same inputs; W: original weights (f64
    numpy); S: oracle statistics; gpu: dict of numpy arrays from the HIP path
    (qweight, scales, zeros, g_idx, optionally w_hat).  Returns a report and
    raises AssertionError on any failure.

    sampled_rows: W and gpu hold a sample of a layer's rows.  A row whose
    trajectory left the oracle's at an excused near-tie is another valid
    GPTQ result with its own error, which a handful of rows cannot average
    out; the layer-error bound then covers the rows that did not diverge
    (the same trajectory), and the diverged rows are bounded in number.
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
    # first divergence of each row, in processing order (d when none)
    first = np.where(mism.any(axis=1), np.argmax(mism, axis=1), d)
    report = dict(mismatch_elems=int(mism.sum()), mismatch_rate=float(mism.mean()),
                  rows_diverged=int(rows_div.size), rows=m)
    problems = []
    if g == -1:
        # fitted on the original weights: identical inputs, exact result
        if not (np.array_equal(zeros, res.zeros) and np.array_equal(scales, res.scales)):
            problems.append("row grid differs")
    else:
        # groups that start before the row's first divergence are unique;
        # a zero-point near-tie at a group start is itself a divergence point
        starts = np.arange(scales.shape[1]) * g
        zmis = zeros != res.zeros
        zfirst = np.where(zmis.any(axis=1), starts[np.argmax(zmis, axis=1)], d)
        first = np.minimum(first, zfirst)
        uniq = starts[None, :] < first[:, None]
        zbad = (zeros != res.zeros) & uniq & (starts[None, :] < zfirst[:, None])
        if zbad.any():
            problems.append(f"zero points differ on {int(zbad.sum())} unique entries")
        rel = np.abs(scales.astype(np.float64) - res.scales) / res.scales
        rel = np.where(uniq, rel, 0.0)
        report["scale_rel_unique"] = float(rel.max(initial=0.0))
        if rel.max(initial=0.0) > SCALE_RTOL:
            problems.append(f"scale rel err {rel.max()}")
    report["rows_diverged"] = int(np.sum(first < d))
    # each row's first divergence must sit on a near-tie of the independent
    # oracle: its pre-rounding value (code) or -lo/Delta (zero point) lies
    # within BAND of a rounding boundary
    bad_first = 0
    for r in np.nonzero(first < d)[0]:
        j = int(first[r])
        near = tie_distance(res.v_perm[r, j]) < BAND
        if g > 0 and j % g == 0:
            near = near or tie_distance(res.zsrc_perm[r, j // g]) < BAND
        bad_first += not near
    report["bad_first_divergence"] = bad_first
    if bad_first:
        problems.append(f"{bad_first} first divergences are not near-ties of the oracle")
    Wp = np.array(W, dtype=np.float64)
    Wp[:, res.dead] = 0.0
    Wp = Wp[:, res.perm]
    rg = (scales[:, 0], zeros[:, 0]) if g == -1 else None
    rep = replay(Wp, res.R, bits, g, b, codes_perm, scales, zeros, rg)
    report.update(forced=rep["forced"], bad_code=rep["bad_code"],
                  bad_zero=rep["bad_zero"], bad_scale=rep["bad_scale"])
    if rep["bad_code"] or rep["bad_zero"] or rep["bad_scale"]:
        problems.append("replay rejects GPU decisions")
    gid = res.g_idx if g > 0 else np.zeros(d, dtype=np.int64)
    rows = np.arange(m)[:, None]
    w_hat_codes = scales[rows, gid[None, :]].astype(np.float64) * \
        (codes_gpu - zeros[rows, gid[None, :]])
    if check_w_hat and "w_hat" in gpu:
        w_hat = np.asarray(gpu["w_hat"], dtype=np.float64)
        if not np.allclose(w_hat, w_hat_codes, rtol=1e-6, atol=0):
            problems.append("w_hat inconsistent with codes/scales/zeros")
    # dequantized weights: unique on each row's prefix before its first
    # divergence (processing order), mapped back to the original columns
    pref = np.zeros((m, d), dtype=bool)
    pref[:, res.perm] = np.arange(d)[None, :] < first[:, None]
    diff = np.where(pref, w_hat_codes - res.w_hat, 0.0)
    ref = np.where(pref, res.w_hat, 0.0)
    rel_w = np.linalg.norm(diff) / max(np.linalg.norm(ref), 1e-30)
    report["unique_frac"] = float(pref.mean())
    report["w_hat_rel_all"] = float(np.linalg.norm(w_hat_codes - res.w_hat) /
                                    max(np.linalg.norm(res.w_hat), 1e-30))
    keep = np.ones(m, dtype=bool)
    if sampled_rows:
        keep = first >= d
        report["rows_compared_for_layer_error"] = int(keep.sum())
        if keep.sum() < max(1, (3 * m) // 4):
            problems.append(f"{m - int(keep.sum())} of {m} sampled rows diverged")
    L_orc = orc.layer_error(W[keep], res.w_hat[keep], S, n) if keep.any() else 0.0
    L_gpu = orc.layer_error(W[keep], w_hat_codes[keep], S, n) if keep.any() else 0.0
    rel_L = abs(L_gpu - L_orc) / max(L_orc, 1e-300)
    report.update(w_hat_rel=float(rel_w), layer_err_rel=float(rel_L),
                  layer_err=float(L_orc))
    if rel_w > 1e-3:
        problems.append(f"||dW_hat||/||W_hat|| = {rel_w}")
    if rel_L > 1e-3:
        problems.append(f"layer error rel diff {rel_L}")
    assert not problems, f"{problems} {report}"
    return report
