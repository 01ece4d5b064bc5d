"""Comparison of the HIP path's outputs with the float64 oracle.

GPTQ's column chain is chaotic: one code that lands on the other side of a
rounding boundary changes every later code in its row, and both outcomes are
correct.  So the comparison has two parts:

1. Unique results are compared directly with the independent oracle run:
   permutation, dead mask, group index, the packing of the GPU's own codes,
   and -- on each row's prefix before its first divergence (a code or a
   zero point that landed on the other side of a near-tie) -- the codes,
   scales, zero points and dequantized weights.  Each first divergence must
   be a near-tie of the independent oracle.  The raw element mismatch rate,
   the number of diverged rows and the unique fraction are reported.
2. The tie-forced oracle: the oracle's loop re-run in float64 from the same
   inputs, which takes the GPU's decision only where the two differ at a
   near-tie (within `band` grid steps of the rounding boundary) and rejects
   any other difference.  It is the independent oracle up to each row's
   first near-tie, and after it the oracle's own continuation of the
   trajectory the tolerance admits.  The whole-layer figures -- dequantized
   weights and layer error, each to 1e-3 relative -- are taken against it.

The replay uses the oracle's primitives (grid fit, encoder); nothing the GPU
produced is an expected value except a decision the band admits.
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
           row_grid=None, band=BAND, symmetric=False, gpos=None):
    """The oracle's column loop, re-run in float64, taking the GPU's decision
    only where the two differ at a near-tie (the "tie-forced oracle").

    At a dynamic group start the replay fits its own grid on its own working
    weights; a GPU zero point that differs must be within `band` of the
    replay's rounding boundary of -lo/Delta (it is then taken), and the GPU
    scale must agree to SCALE_RTOL.  Every GPU code must equal the replay's
    rounding or lie within `band` of its boundary (it is then taken).
    Anything else is counted as a bad decision.  The replay's own values
    q = Delta (c - z), with its own scales, form W_hat_tf: the oracle's
    result on the trajectory the tolerance admits.

    Wp: [m, d] oracle working copy in processing order (dead columns zeroed);
    R: oracle factor; codes_perm: GPU codes (unsigned form) in processing
    order; scales/zeros: GPU [m, n_g] (unsigned zero points); row_grid:
    (scale, zero) for g = -1; gpos: static grids, position j -> group.
    Returns a dict of counts and w_hat_tf [m, d] (processing order).
    """
    W = np.array(Wp, dtype=np.float64, copy=True)
    m, d = W.shape
    maxq = orc.grid_maxq(bits, symmetric)
    bad_code = bad_zero = bad_scale = forced = 0
    w_hat_tf = np.zeros((m, d))
    if group_size == -1:
        scale = np.asarray(row_grid[0], dtype=np.float32)
        zero = np.asarray(row_grid[1], dtype=np.int64)
    for i in range(0, d, blocksize):
        i2 = min(i + blocksize, d)
        E = np.zeros((m, i2 - i))
        for j in range(i, i2):
            if gpos is not None:
                scale = np.asarray(scales[:, gpos[j]], dtype=np.float32)
                zero = np.asarray(zeros[:, gpos[j]], dtype=np.int64)
            elif group_size > 0 and j % group_size == 0:
                grp = W[:, j:min(j + group_size, d)]
                s_r, z_r = orc.fit_grid(grp, bits, symmetric)
                lo32 = np.minimum(grp.min(axis=1), 0.0).astype(np.float32)
                zsrc = (-lo32 / s_r).astype(np.float64)
                g = j // group_size
                zg = np.asarray(zeros[:, g], dtype=np.int64)
                sg = np.asarray(scales[:, g], dtype=np.float32)
                zdiff = zg != z_r
                near = np.zeros(m, dtype=bool) if symmetric else tie_distance(zsrc) < band
                bad_zero += int(np.sum(zdiff & ~near))
                forced += int(np.sum(zdiff & near))
                rel = np.abs(sg.astype(np.float64) - s_r) / s_r
                bad_scale += int(np.sum(rel > SCALE_RTOL))
                scale, zero = s_r, np.where(zdiff & near, zg, z_r)
            c_r, _, v = orc.encode(W[:, j], scale, zero, bits, maxq)
            cg = np.asarray(codes_perm[:, j], dtype=np.int64)
            cdiff = cg != c_r
            # a boundary only separates codes inside [0, maxq]; the band test
            # on v covers both the rounding and the clipping thresholds
            near = tie_distance(v) < band
            bad_code += int(np.sum(cdiff & ~near))
            forced += int(np.sum(cdiff & near))
            c = np.where(cdiff & near, cg, c_r)
            q = scale.astype(np.float64) * (c - zero)
            w_hat_tf[:, j] = q
            eta = (W[:, j] - q) / R[j, j]
            W[:, j:i2] -= eta[:, None] * R[j, j:i2][None, :]
            E[:, j - i] = eta
        W[:, i2:] -= E @ R[i:i2, i2:]
    return dict(bad_code=bad_code, bad_zero=bad_zero, bad_scale=bad_scale,
                forced=forced, maxq=maxq, w_hat_tf=w_hat_tf)


def unpack_gpu(qweight, d, bits):
    return orc.unpack_codes(np.asarray(qweight).view(np.uint32), d, bits)


def unsigned_codes(stored, zeros_used, g_idx, bits, signed):
    """GPU codes in the unsigned form c (stored signed codes are the low bits
    of c - z: sign-extend and add z)."""
    if not signed:
        return stored
    s = np.where(stored >= 2 ** (bits - 1), stored - 2 ** bits, stored)
    return s + zeros_used[np.arange(stored.shape[0])[:, None], g_idx[None, :]]


def compare_layer(res, W, S, n, gpu, params, check_w_hat=True, strict=True):
    """Full comparison of one quantized layer (or a sample of its rows: rows
    are independent given R and their grids).

    res: oracle GPTQResult from the same inputs; W: original weights (f64
    numpy); S: oracle statistics; gpu: dict of numpy arrays from the HIP path
    (qweight, scales, zeros, g_idx, optionally w_hat).  Returns a report and
    raises AssertionError on any failure.

    Whole-layer figures (dequantized weights to 1e-3 in Frobenius norm, the
    layer error (1/N)||(W - W_hat) X||_F^2 to 1e-3) are taken against the
    tie-forced oracle (see ``replay``), which is the independent oracle
    except where the tolerance admits another rounding; the same figures
    against the independent oracle are reported, and enforced on each row's
    prefix before its first divergence.  With strict=False nothing is
    raised: the report lists what failed under "problems".
    """
    bits, g, b = params["bits"], params["group_size"], params["blocksize"]
    symmetric = params.get("grid", "minmax") == "symmetric"
    static = g > 0 and (params.get("static_groups", False) or
                        params.get("grid", "minmax") == "fixed")
    m, d = W.shape
    qweight = np.asarray(gpu["qweight"])
    stored = unpack_gpu(qweight, d, bits)
    # packing is integer work: bit-exact against the oracle's packer
    np.testing.assert_array_equal(orc.pack_codes(stored, bits),
                                  qweight.view(np.uint32))
    np.testing.assert_array_equal(np.asarray(gpu["g_idx"]), res.g_idx)
    scales = np.asarray(gpu["scales"], dtype=np.float32)
    zeros = np.asarray(gpu["zeros"], dtype=np.int64)
    if symmetric:
        # signed codes: the stored zero point is 0, the grid's own is h
        assert np.all(zeros == 0), "signed codes must come with zero points 0"
        zeros = np.full_like(zeros, 2 ** (bits - 1) - 1)
    codes_gpu = unsigned_codes(stored, zeros, res.g_idx, bits, symmetric)
    assert scales.shape == res.scales.shape and zeros.shape == res.zeros.shape
    codes_perm = codes_gpu[:, res.perm]
    mism = codes_perm != res.codes_perm
    rows_div = np.nonzero(mism.any(axis=1))[0]
    # first divergence of each row, in processing order (d when none)
    first = np.where(mism.any(axis=1), np.argmax(mism, axis=1), d)
    report = dict(mismatch_elems=int(mism.sum()), mismatch_rate=float(mism.mean()),
                  rows_diverged=int(rows_div.size), rows=m)
    problems = []
    if g == -1 or static:
        # fitted on the original weights (or given): identical inputs, exact
        if not (np.array_equal(zeros, res.zeros) and np.array_equal(scales, res.scales)):
            problems.append("row / static grid differs")
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
        if g > 0 and not static and j % g == 0:
            near = near or tie_distance(res.zsrc_perm[r, j // g]) < BAND
        bad_first += not near
    report["bad_first_divergence"] = bad_first
    if bad_first:
        problems.append(f"{bad_first} first divergences are not near-ties of the oracle")
    Wp = np.array(W, dtype=np.float64)
    Wp[:, res.dead] = 0.0
    Wp = Wp[:, res.perm]
    rg = (scales[:, 0], zeros[:, 0]) if g == -1 else None
    gpos = res.perm // g if static else None
    rep = replay(Wp, res.R, bits, g, b, codes_perm, scales, zeros, rg,
                 symmetric=symmetric, gpos=gpos)
    report.update(forced=rep["forced"], bad_code=rep["bad_code"],
                  bad_zero=rep["bad_zero"], bad_scale=rep["bad_scale"])
    if rep["bad_code"] or rep["bad_zero"] or rep["bad_scale"]:
        problems.append("replay rejects GPU decisions")
    w_hat_tf = np.empty((m, d))
    w_hat_tf[:, res.perm] = rep["w_hat_tf"]
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
    # whole layer against the tie-forced oracle
    rel_w_tf = np.linalg.norm(w_hat_codes - w_hat_tf) / max(np.linalg.norm(w_hat_tf), 1e-30)
    L_tf = orc.layer_error(W, w_hat_tf, S, n)
    L_gpu = orc.layer_error(W, w_hat_codes, S, n)
    L_orc = orc.layer_error(W, res.w_hat, S, n)
    rel_L = abs(L_gpu - L_tf) / max(L_tf, 1e-300)
    report.update(w_hat_rel=float(rel_w), w_hat_rel_tf=float(rel_w_tf),
                  layer_err_rel=float(rel_L), layer_err=float(L_tf),
                  layer_err_rel_signed=float((L_gpu - L_tf) / max(L_tf, 1e-300)),
                  layer_err_independent=float(L_orc),
                  layer_err_rel_independent=float(abs(L_gpu - L_orc) / max(L_orc, 1e-300)),
                  w_hat_dnorm2_tf=float(np.sum((w_hat_codes - w_hat_tf) ** 2)),
                  w_hat_norm2_tf=float(np.sum(w_hat_tf ** 2)))
    if rel_w > 1e-3:
        problems.append(f"||dW_hat||/||W_hat|| on unique prefixes = {rel_w}")
    if rel_w_tf > 1e-3:
        problems.append(f"||W_hat - W_hat_tf||/||W_hat_tf|| = {rel_w_tf}")
    if rel_L > 1e-3:
        problems.append(f"layer error rel diff {rel_L}")
    report["problems"] = problems
    assert not (strict and problems), f"{problems} {report}"
    return report
