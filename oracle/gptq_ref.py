"""GPTQ layer quantization, written plainly in float64 NumPy/SciPy.

TEST INFRASTRUCTURE ONLY -- see the package docstring.  This module is the
correctness reference the HIP path is compared against; it is slow on purpose
and follows the pages' steps in their order and notation.

Page shorthand used below:
  [derivation]  hbblog.cn, "GPTQ 从零推导" (equations numbered (1)-(68))
  [teardown]    pinghaoyang.com.cn, "GPTQ 完全拆解" (toy OBS example, Algorithm 1)

Readings taken where the pages are silent (both sides implement the same
reading independently; "parity unpinned" = no page fixes a value for it):

  * H scale: H = (2/N) X X^T ([derivation] eq. (9)).  The toy example of
    [teardown] uses 2 X X^T; the helpers for it take H directly.
  * Rounding: round half to even (numpy ``rint``).            parity unpinned
  * Grid fit (min-max, [derivation] section 1.1): Delta = (hi - lo) /
    (2^b - 1), z = rint(-lo / Delta) (pinned: a range whose -lo/Delta has a
    fractional part above 1/2).  Our readings on top: the range is widened
    to contain 0 so the zero point represents 0 exactly; an all-zero range
    is replaced by [-1, 1]; the fit is evaluated in float32, the precision
    the scales are stored and the kernel decides the integer zero point
    in.                                                         parity unpinned
  * group_size = -1: one grid per row, fitted once on the ORIGINAL row before
    dead columns are zeroed ([derivation] section 10 pseudocode order).
  * group_size > 0: dynamic groups -- refitted at each group start, in
    processing order, on the current working weights ([derivation] 8.3/8.4);
    group_id[perm[j]] = j // g.                                 parity unpinned
  * Symmetric grid ([derivation] 1.1 names symmetric grids, 8.4 the signed
    code form): range [-a, a], a = max|w| (0 in range), 2^b - 1 levels
    -h..h with h = 2^(b-1) - 1, Delta = a / h; codes stored signed (c - h)
    in b-bit two's complement.  At b = 2 this is the ternary grid
    {-1, 0, +1} Delta of [teardown] "extreme quantization".  parity unpinned
  * Static groups ([derivation] 8.3): each group's grid is fitted before
    GPTQ on the ORIGINAL contiguous columns of the original row (dead
    columns included, like the whole-row grid); processing position j uses
    group floor(perm[j] / g); group_id is then the trivial k // g.
  * A group start must see fully compensated columns: every group that starts
    inside a block must end inside it.  Other (g, blocksize) pairs are
    rejected.                                                  parity unpinned
  * Damping floor: 2^-23 (float32 machine epsilon, the pseudocode's
    ``finfo(H.dtype).eps`` for a float32 H).
  * Cholesky failure: damp *= 10, at most 5 retries ([derivation] section 10
    says only "raise the damping and retry").                  parity unpinned
  * Packing: per row, an LSB-first bit stream of b-bit codes in little-endian
    uint32 words, row stride ceil(d*b/32) words.               parity unpinned
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import scipy.linalg as sla

__all__ = [
    "EPS_FLOOR", "MAX_RETRIES", "NotSPDError",
    "hessian_sum", "hessian_from_sum", "fit_grid", "encode", "prepare",
    "factor", "check_group_layout", "quantize_columns", "gptq_layer",
    "pack_codes", "unpack_codes", "layer_error", "proxy_loss",
    "obs_criterion", "obs_update", "kkt_update", "downdate",
    "block_update", "rtn", "GPTQResult", "grid_maxq",
    "static_group_grids", "stored_codes", "dequantize", "dequant_matmul",
    "bf16_round", "activate", "gptq_stack",
]

EPS_FLOOR = 2.0 ** -23      # damping floor: float32 machine epsilon
MAX_RETRIES = 5             # Cholesky retries, damping x10 each time


class NotSPDError(RuntimeError):
    """The damped Hessian stayed non positive-definite after all retries."""


# ----------------------------------------------------------------------------
# Statistics: [derivation] section 2, eq. (5) and eq. (9)
# ----------------------------------------------------------------------------

def hessian_sum(X_tok, chunk: int = 16384) -> np.ndarray:
    """S = sum_t x_t x_t^T for token-major activations X_tok [N, d].

    X = reshape(A, [N, d])^T is the pages' [d, N] matrix (eq. (5)); S = X X^T.
    Accumulated in float64 over token chunks ("can be accumulated in batches",
    [derivation] 9.4).  Any float input dtype converts exactly to float64.
    """
    X_tok = np.asarray(X_tok)
    n, d = X_tok.shape
    S = np.zeros((d, d), dtype=np.float64)
    for t0 in range(0, n, chunk):
        Xc = np.asarray(X_tok[t0:t0 + chunk], dtype=np.float64)
        S += Xc.T @ Xc
    return S


def hessian_from_sum(S, n: int) -> np.ndarray:
    """H = (2/N) X X^T, [derivation] eq. (9)."""
    return (2.0 / float(n)) * np.asarray(S, dtype=np.float64)


# ----------------------------------------------------------------------------
# The b-bit affine quantizer: [derivation] section 1.1 and eq. (36)
# ----------------------------------------------------------------------------

def grid_maxq(bits: int, symmetric: bool = False) -> int:
    """Largest unsigned code: 2^b - 1 for the min-max grid; 2^b - 2 for the
    symmetric grid, whose 2^b - 1 levels -h..h (h = 2^(b-1) - 1) sit
    symmetrically around an exact 0 (at b = 2 the ternary grid {-1, 0, +1})."""
    return 2 ** bits - 2 if symmetric else 2 ** bits - 1


def fit_grid(w, bits: int, symmetric: bool = False):
    """Min-max grid per row of w [m, k]: returns (scale float32 [m], zero [m]).

    Follows the rough min-max fit of [derivation] 1.1 with 15 -> 2^b - 1,
    widened to contain 0 (so the integer zero point represents 0 exactly) and
    with an all-zero range mapped to [-1, 1].  Evaluated in float32.

    symmetric: the symmetric grid that [derivation] 1.1 names (its 8.4 notes
    the signed code form): the range becomes [-a, a] with a = max |w|, the
    levels are 2^b - 1 (maxq = 2^b - 2), so Delta = a / h and z = h with
    h = 2^(b-1) - 1; the extremes +-a land exactly on the outer levels.
    """
    w = np.asarray(w)
    if w.ndim == 1:
        w = w[:, None]
    maxq = np.float32(2 ** bits - 1)
    lo = np.minimum(w.min(axis=1), 0.0).astype(np.float32)
    hi = np.maximum(w.max(axis=1), 0.0).astype(np.float32)
    if symmetric:
        maxq = np.float32(grid_maxq(bits, True))
        hi = np.maximum(-lo, hi)
        lo = -hi
    flat = hi == lo
    lo = np.where(flat, np.float32(-1.0), lo).astype(np.float32)
    hi = np.where(flat, np.float32(1.0), hi).astype(np.float32)
    scale = ((hi - lo) / maxq).astype(np.float32)
    zero = np.rint((-lo) / scale).astype(np.float32)
    zero = np.clip(zero, np.float32(0), maxq)
    return scale, zero.astype(np.int64)


def encode(w, scale, zero, bits: int, maxq=None):
    """c = clip(round(w/Delta) + z, 0, 2^b-1), q = Delta (c - z)   (eq. (36)).

    Returns (c int64, q float64, v float64) where v = w / Delta is the
    pre-rounding value (used to tell a genuine mismatch from a near-tie).
    ``maxq`` overrides the top code (the symmetric grid stops at 2^b - 2).
    """
    if maxq is None:
        maxq = 2 ** bits - 1
    scale = np.asarray(scale, dtype=np.float64)
    zero = np.asarray(zero, dtype=np.float64)
    v = np.asarray(w, dtype=np.float64) / scale
    c = np.clip(np.rint(v) + zero, 0, maxq)
    q = scale * (c - zero)
    return c.astype(np.int64), q, v


# ----------------------------------------------------------------------------
# Pre-processing: dead features, act-order, damping ([derivation] section 10,
# 8.3 eq. (34), 2.6 eq. (12))
# ----------------------------------------------------------------------------

def prepare(S, n: int, percdamp: float, act_order: bool, damp_override=None):
    """Return (H_perm, perm, dead, damp) with H_perm still UNDAMPED.

    * dead = unseen input features (zero diagonal); their diagonal becomes 1
      (the working weights of those columns are zeroed in ``gptq_layer``).
    * perm = identity, or the stable argsort of diag(H) in descending order
      (act-order), taken after the dead fix; H is permuted on both sides.
    * damp = max(percdamp * mean(diag H), 2^-23) unless overridden.
    """
    H = hessian_from_sum(S, n).copy()
    d = H.shape[0]
    dead = np.diag(H) == 0.0
    idx = np.nonzero(dead)[0]
    H[idx, idx] = 1.0
    if act_order:
        perm = np.argsort(-np.diag(H), kind="stable")
    else:
        perm = np.arange(d)
    H = H[np.ix_(perm, perm)]
    if damp_override is None:
        damp = max(percdamp * float(np.mean(np.diag(H))), EPS_FLOOR)
    else:
        damp = float(damp_override)
    return H, perm, dead, damp


def factor(H, damp: float, max_retries: int = MAX_RETRIES):
    """R = upper Cholesky factor of (H + damp I)^-1, the route of [derivation]
    section 10: L = chol(H), G = cholesky_inverse(L), G = (G + G^T)/2,
    R = chol_upper(G).  G = R^T R (eq. (37)).

    On a failed factorisation the damping is multiplied by 10 and the whole
    route is retried.  Returns (R, damp_used); raises NotSPDError.
    """
    H = np.asarray(H, dtype=np.float64)
    d = H.shape[0]
    eye = np.eye(d)
    for _ in range(max_retries + 1):
        Hd = H + damp * eye
        try:
            if not np.all(np.isfinite(Hd)):
                raise np.linalg.LinAlgError("non-finite")
            L = np.linalg.cholesky(Hd)
            Linv = sla.solve_triangular(L, eye, lower=True)
            G = Linv.T @ Linv
            G = 0.5 * (G + G.T)
            R = np.linalg.cholesky(G).T
            if not np.all(np.isfinite(R)):
                raise np.linalg.LinAlgError("non-finite factor")
            return R, damp
        except np.linalg.LinAlgError:
            damp *= 10.0
    raise NotSPDError(f"not positive definite; last damp tried {damp / 10.0}")


# ----------------------------------------------------------------------------
# Column loop with lazy block updates ([teardown] Algorithm 1;
# [derivation] eq. (42), (45), (46) and the section 10 pseudocode)
# ----------------------------------------------------------------------------

def check_group_layout(d: int, group_size: int, blocksize: int) -> bool:
    """True when every dynamic group starts on fully compensated columns.

    A group starting at processing position j is fitted on W_work[:, j:j+g]
    at the moment column j is reached.  Columns past the current block have
    not yet received the deferred updates of this block's earlier columns, so
    a group starting inside a block must end inside it.
    """
    if group_size == -1:
        return True
    if group_size <= 0 or blocksize <= 0:
        return False
    for j in range(0, d, group_size):
        off = j % blocksize
        if off != 0 and off + min(group_size, d - j) > blocksize:
            return False
    return True


@dataclass
class GPTQResult:
    codes: np.ndarray           # [m, d] int64, ORIGINAL column order
    scales: np.ndarray          # [m, n_g] float32 (processing-group order)
    zeros: np.ndarray           # [m, n_g] int64
    g_idx: np.ndarray           # [d] int64, group of each original column
    w_hat: np.ndarray           # [m, d] float64, ORIGINAL column order
    perm: np.ndarray            # [d] processing order -> original column
    dead: np.ndarray            # [d] bool, original order
    damp: float
    R: np.ndarray               # [d, d] upper factor (processing order)
    codes_perm: np.ndarray = field(repr=False, default=None)   # [m, d]
    v_perm: np.ndarray = field(repr=False, default=None)       # w/Delta
    eta_perm: np.ndarray = field(repr=False, default=None)     # rho / R_jj
    rho_perm: np.ndarray = field(repr=False, default=None)     # w - q
    zsrc_perm: np.ndarray = field(repr=False, default=None)    # -lo/Delta at fits
    packed: np.ndarray = field(repr=False, default=None)       # [m, words]
    signed: bool = False        # symmetric grid: stored codes are c - z


def quantize_columns(Wp, R, bits: int, group_size: int, blocksize: int,
                     row_grid=None, symmetric: bool = False, static_grid=None):
    """The blocked GPTQ column loop on a working copy already in processing
    order (dead columns zeroed).

    For each block [i, i2): for each column j in it, fit the group grid if j
    starts a group, encode the column, rho = w - q, eta = rho / R_jj, update
    W[:, j:i2] -= eta R[j, j:i2]; then W[:, i2:] -= E R[i:i2, i2:].

    symmetric: dynamic refits use the symmetric grid (see ``fit_grid``).
    static_grid: (scales [m, n_s], zeros [m, n_s], gpos [d]) grids fixed in
    advance (static groups, [derivation] 8.3): processing position j uses
    column gpos[j] of them and nothing is refitted.

    Returns dict with codes, q, v, eta, rho (all [m, d], processing order),
    scales [m, n_g], zeros [m, n_g], zsrc [m, n_g] (the unrounded -lo/Delta).
    """
    W = np.array(Wp, dtype=np.float64, copy=True)
    R = np.asarray(R, dtype=np.float64)
    m, d = W.shape
    maxq = grid_maxq(bits, symmetric)
    if static_grid is None and not check_group_layout(d, group_size, blocksize):
        raise ValueError("group_size / blocksize combination not supported")
    n_g = 1 if group_size == -1 else -(-d // group_size)
    codes = np.zeros((m, d), dtype=np.int64)
    Q = np.zeros((m, d))
    V = np.zeros((m, d))
    ETA = np.zeros((m, d))
    RHO = np.zeros((m, d))
    scales = np.zeros((m, n_g), dtype=np.float32)
    zeros = np.zeros((m, n_g), dtype=np.int64)
    zsrc = np.zeros((m, n_g))
    if static_grid is not None:
        scales = np.array(static_grid[0], dtype=np.float32)
        zeros = np.array(static_grid[1], dtype=np.int64)
        gpos = np.asarray(static_grid[2], dtype=np.int64)
        zsrc = zeros.astype(np.float64)     # zero points are given, not rounded
    elif group_size == -1:
        scale, zero = row_grid
        scales[:, 0] = scale
        zeros[:, 0] = zero
    for i in range(0, d, blocksize):
        i2 = min(i + blocksize, d)
        E = np.zeros((m, i2 - i))
        for j in range(i, i2):
            if static_grid is not None:
                scale, zero = scales[:, gpos[j]], zeros[:, gpos[j]]
            elif group_size > 0 and j % group_size == 0:
                grp = W[:, j:min(j + group_size, d)]
                scale, zero = fit_grid(grp, bits, symmetric)
                lo32 = np.minimum(grp.min(axis=1), 0.0).astype(np.float32)
                zsrc[:, j // group_size] = (-lo32 / scale).astype(np.float64)
                if symmetric:       # z = h is fixed: no rounding decides it
                    zsrc[:, j // group_size] = zero
                scales[:, j // group_size] = scale
                zeros[:, j // group_size] = zero
            c, q, v = encode(W[:, j], scale, zero, bits, maxq)
            rho = W[:, j] - q
            eta = rho / R[j, j]
            W[:, j:i2] -= eta[:, None] * R[j, j:i2][None, :]
            E[:, j - i] = eta
            codes[:, j] = c
            Q[:, j] = q
            V[:, j] = v
            ETA[:, j] = eta
            RHO[:, j] = rho
        W[:, i2:] -= E @ R[i:i2, i2:]
    return dict(codes=codes, q=Q, v=V, eta=ETA, rho=RHO, scales=scales,
                zeros=zeros, zsrc=zsrc)


def static_group_grids(W, bits: int, group_size: int, symmetric: bool = False):
    """Grids of the static groups: fitted before GPTQ on the ORIGINAL
    contiguous columns [G g, (G+1) g) of every row ([derivation] 8.3),
    like the whole-row grid on the original row.  Returns ([m, n_g] scales,
    [m, n_g] zeros)."""
    W = np.asarray(W, dtype=np.float64)
    m, d = W.shape
    n_g = -(-d // group_size)
    scales = np.zeros((m, n_g), dtype=np.float32)
    zeros = np.zeros((m, n_g), dtype=np.int64)
    for G in range(n_g):
        scales[:, G], zeros[:, G] = fit_grid(W[:, G * group_size:(G + 1) * group_size],
                                             bits, symmetric)
    return scales, zeros


def gptq_layer(W, S, n: int, bits: int = 4, group_size: int = -1,
               blocksize: int = 128, percdamp: float = 0.01,
               act_order: bool = False, damp_override=None,
               fixed_grid=None, symmetric: bool = False,
               static_groups: bool = False) -> GPTQResult:
    """Quantize one linear layer W [m, d] given S = X X^T over n tokens.

    The steps and their order are the [derivation] section 10 pseudocode,
    extended to b bits, dynamic groups and act-order as its sections 8.3-8.4
    describe.  ``fixed_grid`` = (scale[m], zero[m]) replaces the row fit
    (the section 11 worked example fixes its grid in advance); with
    group_size > 0 it is (scales[m, n_g], zeros[m, n_g]) on the static
    group layout.  ``symmetric`` selects the symmetric grid with signed
    codes (``fit_grid``); ``static_groups`` fits the groups once on the
    original contiguous columns ([derivation] 8.3) instead of refitting
    them in processing order.
    """
    W = np.asarray(W, dtype=np.float64)
    m, d = W.shape
    if bits not in (2, 3, 4, 8):
        raise ValueError("bits must be 2, 3, 4 or 8")
    if group_size == 0 or group_size < -1 or blocksize < 1:
        raise ValueError("bad group_size / blocksize")
    if fixed_grid is not None and symmetric:
        raise ValueError("a fixed grid carries its own zero points")
    static = group_size > 0 and (static_groups or fixed_grid is not None)
    # whole-row grid is fitted on the original row, before the dead fix
    if group_size == -1:
        row_grid = fixed_grid if fixed_grid is not None else fit_grid(W, bits, symmetric)
    else:
        row_grid = None
    if static:
        sg = fixed_grid if fixed_grid is not None else \
            static_group_grids(W, bits, group_size, symmetric)
    H, perm, dead, damp = prepare(S, n, percdamp, act_order, damp_override)
    R, damp = factor(H, damp)
    Wp = W.copy()
    Wp[:, dead] = 0.0
    Wp = Wp[:, perm]
    if static:
        out = quantize_columns(Wp, R, bits, group_size, blocksize,
                               symmetric=symmetric,
                               static_grid=(sg[0], sg[1], perm // group_size))
    else:
        out = quantize_columns(Wp, R, bits, group_size, blocksize, row_grid,
                               symmetric=symmetric)
    codes = np.empty_like(out["codes"])
    codes[:, perm] = out["codes"]
    w_hat = np.empty((m, d))
    w_hat[:, perm] = out["q"]
    g_idx = np.zeros(d, dtype=np.int64)
    if static:
        g_idx = np.arange(d) // group_size
    elif group_size > 0:
        g_idx[perm] = np.arange(d) // group_size
    res = GPTQResult(codes=codes, scales=out["scales"], zeros=out["zeros"],
                     g_idx=g_idx, w_hat=w_hat, perm=perm, dead=dead,
                     damp=damp, R=R, codes_perm=out["codes"],
                     v_perm=out["v"], eta_perm=out["eta"],
                     rho_perm=out["rho"], zsrc_perm=out["zsrc"],
                     packed=pack_codes(codes, bits), signed=symmetric)
    if symmetric:
        res.packed = pack_codes(stored_codes(res, bits), bits)
    return res


def stored_codes(res: "GPTQResult", bits: int) -> np.ndarray:
    """The codes as stored: unsigned c for the min-max and fixed grids; for
    the symmetric grid the signed code c - z ([derivation] 8.4: the same
    levels written as -h..h), kept as its low b bits (two's complement)."""
    if not res.signed:
        return res.codes
    z = res.zeros[np.arange(res.codes.shape[0])[:, None], res.g_idx[None, :]]
    return np.mod(res.codes - z, 2 ** bits)


# ----------------------------------------------------------------------------
# Output format ([derivation] 3.1: codes are stored packed, layout left to the
# kernel -- our reading: LSB-first bit stream per row in uint32 words)
# ----------------------------------------------------------------------------

def pack_codes(codes, bits: int) -> np.ndarray:
    """Pack integer codes [m, d] into uint32 words [m, ceil(d*bits/32)].

    Column c of a row occupies stream bits [c*bits, (c+1)*bits); stream bit p
    is bit (p % 32) of word p // 32.  Unused trailing bits are zero.
    """
    codes = np.asarray(codes, dtype=np.int64)
    m, d = codes.shape
    words = -(-d * bits // 32)
    stream = np.zeros((m, words * 32), dtype=np.uint64)
    for k in range(bits):
        stream[:, np.arange(d) * bits + k] = (codes >> k) & 1
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    out = (stream.reshape(m, words, 32) * weights).sum(axis=2)
    return out.astype(np.uint32)


def unpack_codes(packed, d: int, bits: int) -> np.ndarray:
    """Inverse of ``pack_codes``."""
    packed = np.asarray(packed, dtype=np.uint64)
    m = packed.shape[0]
    codes = np.zeros((m, d), dtype=np.int64)
    for k in range(bits):
        p = np.arange(d) * bits + k
        bit = (packed[:, p // 32] >> (p % 32).astype(np.uint64)) & np.uint64(1)
        codes |= bit.astype(np.int64) << k
    return codes


# ----------------------------------------------------------------------------
# Inference on the stored format: the dequantized matmul ([wiki] "inference":
# the packed low-bit weights are dequantized inside the matmul kernel;
# [derivation] 3.1 and 8.3: codes, a scale and zero per (row, group), and a
# group id per column when groups and act-order meet)
# ----------------------------------------------------------------------------

def dequantize(packed, scales, zeros, g_idx, d: int, bits: int,
               signed: bool = False) -> np.ndarray:
    """W_hat[r][c] = Delta[r][g(c)] (c_rc - z[r][g(c)]) with g(c) = g_idx[c].

    ``signed``: the stored codes are the low ``bits`` bits of c - z (the
    symmetric grid); they are sign-extended and the zero point is 0."""
    codes = unpack_codes(packed, d, bits)
    scales = np.asarray(scales, dtype=np.float64)
    zeros = np.asarray(zeros, dtype=np.float64)
    g_idx = np.asarray(g_idx, dtype=np.int64)
    rows = np.arange(codes.shape[0])[:, None]
    if signed:
        codes = np.where(codes >= 2 ** (bits - 1), codes - 2 ** bits, codes)
        zeros = np.zeros_like(zeros)
    return scales[rows, g_idx[None, :]] * (codes - zeros[rows, g_idx[None, :]])


def dequant_matmul(x, packed, scales, zeros, g_idx, bits: int,
                   signed: bool = False) -> np.ndarray:
    """Y = x W_hat^T for token-major activations x [n, d]: the layer's
    output on the quantized weights, in float64."""
    x = np.asarray(x, dtype=np.float64)
    W_hat = dequantize(packed, scales, zeros, g_idx, x.shape[1], bits, signed)
    return x @ W_hat.T


# ----------------------------------------------------------------------------
# Layer by layer: [derivation] 3.2 steps 1-2 and 10 (capture each layer's
# inputs, quantize it, check its reconstruction error, go on to the next);
# [teardown] "layer-wise quantization".  Reading: the next layer's inputs are
# the quantized layer's outputs (after an elementwise activation), stored as
# bf16 like any captured activation.
# ----------------------------------------------------------------------------

def bf16_round(y) -> np.ndarray:
    """Round to bfloat16 (8 significant bits, half to even), from float64
    directly (one rounding)."""
    y = np.asarray(y, dtype=np.float64)
    mant, expo = np.frexp(y)                   # y = mant 2^expo, 0.5 <= |mant| < 1
    return np.ldexp(np.rint(mant * 256.0) / 256.0, expo)


def activate(y, activation: str) -> np.ndarray:
    """The elementwise activation between layers: none, relu or silu."""
    y = np.asarray(y, dtype=np.float64)
    if activation == "relu":
        return np.maximum(y, 0.0)
    if activation == "silu":
        return y / (1.0 + np.exp(-y))
    if activation != "none":
        raise ValueError(activation)
    return y


def gptq_stack(Ws, X0, layer_params, activation: str = "none"):
    """Quantize a stack of linear layers in order.  Layer l sees the token-
    major inputs X_l (X_0 given); its statistics, factor and loop are
    ``gptq_layer``; its reconstruction error (1/N)||(W - W_hat) X||_F^2 is
    reported; X_{l+1} = bf16(act(X_l W_hat_l^T)) from the stored format.
    Returns (per-layer list of dicts with res / err / S / X, final X)."""
    X = np.asarray(X0, dtype=np.float64)
    out = []
    for W, p in zip(Ws, layer_params):
        W = np.asarray(W, dtype=np.float64)
        n = X.shape[0]
        S = hessian_sum(X)
        res = gptq_layer(W, S, n, **p)
        err = layer_error(W, res.w_hat, S, n)
        zeros = np.zeros_like(res.zeros) if res.signed else res.zeros
        Y = dequant_matmul(X, res.packed, res.scales, zeros, res.g_idx,
                           p.get("bits", 4), res.signed)
        out.append(dict(res=res, err=err, S=S, X=X))
        X = bf16_round(activate(Y, activation))
    return out, X


# ----------------------------------------------------------------------------
# Diagnostics: [derivation] eq. (6), eq. (43)
# ----------------------------------------------------------------------------

def layer_error(W, W_hat, S, n: int) -> float:
    """(1/N) ||W X - W_hat X||_F^2 = (1/N) sum_r dw_r^T S dw_r   (eq. (6))."""
    dW = np.asarray(W, dtype=np.float64) - np.asarray(W_hat, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    return float(np.einsum("rd,de,re->", dW, S, dW, optimize=True) / float(n))


def proxy_loss(rho_perm, R) -> float:
    """sum over rows and columns of rho^2 / (2 R_jj^2)   (eq. (43))."""
    rjj = np.diag(np.asarray(R, dtype=np.float64))
    return float(np.sum(np.asarray(rho_perm) ** 2 / (2.0 * rjj[None, :] ** 2)))


# ----------------------------------------------------------------------------
# Single- and multi-coordinate OBS helpers used only by the pins
# ([teardown] toy example; [derivation] eq. (22), (23), (26), (30), (31))
# ----------------------------------------------------------------------------

def obs_criterion(w, quant_w, H) -> np.ndarray:
    """Greedy OBS/OBQ score (quant(w_q) - w_q)^2 / [H^-1]_qq for every q."""
    Hinv = np.linalg.inv(np.asarray(H, dtype=np.float64))
    err = np.asarray(quant_w, dtype=np.float64) - np.asarray(w, dtype=np.float64)
    return err ** 2 / np.diag(Hinv)


def obs_update(G_F, p: int, rho: float):
    """delta* = -rho_p / [G_F]_pp * (G_F)[:, p] and its cost rho^2/(2 G_pp)
    (eq. (22), (23))."""
    G_F = np.asarray(G_F, dtype=np.float64)
    delta = -rho / G_F[p, p] * G_F[:, p]
    return delta, rho ** 2 / (2.0 * G_F[p, p])


def kkt_update(H_F, p: int, rho: float):
    """Solve the equality-constrained QP min 1/2 d^T H d s.t. d_p = -rho
    directly from its KKT linear system (the [derivation] 4.4 system)."""
    H_F = np.asarray(H_F, dtype=np.float64)
    k = H_F.shape[0]
    K = np.zeros((k + 1, k + 1))
    K[:k, :k] = H_F
    K[:k, k] = 0.0
    K[p, k] = 1.0
    K[k, p] = 1.0
    rhs = np.zeros(k + 1)
    rhs[k] = -rho
    sol = np.linalg.solve(K, rhs)
    delta = sol[:k]
    return delta, 0.5 * delta @ H_F @ delta


def downdate(G_F, p: int) -> np.ndarray:
    """Inverse Hessian of the remaining coordinates after freezing p,
    G_T = G_TT - G_Tp G_pT / G_pp   (eq. (26))."""
    G_F = np.asarray(G_F, dtype=np.float64)
    keep = [i for i in range(G_F.shape[0]) if i != p]
    Gt = G_F - np.outer(G_F[:, p], G_F[p, :]) / G_F[p, p]
    return Gt[np.ix_(keep, keep)]


def block_update(G_F, B, a_B):
    """Multi-constraint OBS: Gamma = (G_F)_BB, y = Gamma^-1 a_B,
    delta* = (G_F)_{:,B} y, cost = a_B^T y / 2, and the next inverse
    G_T = G_TT - G_TB Gamma^-1 G_BT   (eq. (29)-(31))."""
    G_F = np.asarray(G_F, dtype=np.float64)
    B = list(B)
    T = [i for i in range(G_F.shape[0]) if i not in B]
    Gamma = G_F[np.ix_(B, B)]
    y = np.linalg.solve(Gamma, np.asarray(a_B, dtype=np.float64))
    delta = G_F[:, B] @ y
    cost = 0.5 * float(np.asarray(a_B) @ y)
    Z = np.linalg.solve(Gamma, G_F[np.ix_(B, T)])
    G_T = G_F[np.ix_(T, T)] - G_F[np.ix_(T, B)] @ Z
    return dict(Gamma=Gamma, y=y, delta=delta, cost=cost, G_T=G_T)


def rtn(W, scale, zero, bits: int):
    """Round-to-nearest baseline: encode every weight with no compensation."""
    c, q, _ = encode(np.asarray(W, dtype=np.float64),
                     np.asarray(scale)[:, None], np.asarray(zero)[:, None],
                     bits)
    return c, q
