"""Pins of the float64 oracle to identities the mathematics fixes.

Seeded random tiny layers; every check is against an independent route (a
KKT solve, a closed form, brute force, a reduction to round-to-nearest) or an
exact identity proven on the pages -- never a re-typing of the oracle's own
formula.
"""

import itertools

import numpy as np
import pytest

import oracle as orc


def rand_spd(rng, k, cond_decay=0.5):
    Q, _ = np.linalg.qr(rng.standard_normal((k, k)))
    ev = np.exp(-cond_decay * np.arange(k)) + 0.05
    return (Q * ev) @ Q.T


def rand_layer(rng, m, d, n, rank=None):
    A = rng.standard_normal((d, rank or d))
    Z = rng.standard_normal((rank or d, n))
    X = A @ Z                                  # [d, N]
    W = 0.02 * rng.standard_normal((m, d))
    return W, X.T.copy()                       # token-major activations


@pytest.mark.parametrize("seed", range(5))
def test_obs_update_equals_kkt_solve(seed):
    """eq. (22)/(23) against a direct solve of the KKT system of the
    equality-constrained QP ([derivation] 4.4)."""
    rng = np.random.default_rng(seed)
    k = 6
    H = rand_spd(rng, k)
    for p in range(k):
        rho = rng.standard_normal()
        d1, c1 = orc.obs_update(np.linalg.inv(H), p, rho)
        d2, c2 = orc.kkt_update(H, p, rho)
        np.testing.assert_allclose(d1, d2, atol=1e-10)
        assert abs(c1 - c2) < 1e-10
        assert abs(d1[p] + rho) < 1e-12          # constraint met exactly
        assert c1 >= 0


@pytest.mark.parametrize("seed", range(3))
def test_downdate_is_inverse_of_submatrix(seed):
    """eq. (26): the downdated inverse equals inv(H with p removed)."""
    rng = np.random.default_rng(seed)
    H = rand_spd(rng, 7)
    for p in range(7):
        keep = [i for i in range(7) if i != p]
        np.testing.assert_allclose(orc.downdate(np.linalg.inv(H), p),
                                   np.linalg.inv(H[np.ix_(keep, keep)]),
                                   atol=1e-9)


@pytest.mark.parametrize("seed", range(3))
def test_block_formula_equals_sequential_and_lazy(seed):
    """eq. (32) (block entry -> exit) = sequential single-column OBS updates
    = the Cholesky form with the lazy tail E R_BT (eq. (47)-(49))."""
    rng = np.random.default_rng(seed)
    m, d, b = 5, 9, 4
    H = rand_spd(rng, d)
    R, _ = orc.factor(H, 0.0)
    G = np.linalg.inv(H)
    Win = rng.standard_normal((m, d))
    scale = np.full(m, 0.3, dtype=np.float32)
    zero = np.full(m, 8, dtype=np.int64)
    # sequential single-coordinate OBS with explicit downdates (no Cholesky)
    Wseq = Win.copy()
    Gcur = G.copy()
    Qb = np.zeros((m, b))
    for j in range(b):
        _, q, _ = orc.encode(Wseq[:, j], scale, zero, 4)
        Qb[:, j] = q
        rho = Wseq[:, j] - q
        for r in range(m):
            delta, _ = orc.obs_update(Gcur, 0, rho[r])
            Wseq[r, j:] += delta
        Gcur = orc.downdate(Gcur, 0)
    # block formula (32) from the block-entry state
    D = Win[:, :b] - Qb
    Gamma = G[:b, :b]
    Wblk = Win - D @ np.linalg.solve(Gamma, G[:b, :])
    np.testing.assert_allclose(Wblk, Wseq, atol=1e-10)
    np.testing.assert_allclose(Wblk[:, :b], Qb, atol=1e-10)
    # Cholesky loop with the lazy tail
    out = orc.quantize_columns(Win, R, 4, -1, b, (scale, zero))
    Wtail = Win.copy()
    E = out["eta"][:, :b]
    np.testing.assert_allclose(D, E @ R[:b, :b], atol=1e-10)      # eq. (47)
    Wtail[:, b:] -= E @ R[:b, b:]                                 # eq. (46)
    np.testing.assert_allclose(Wtail[:, b:], Wseq[:, b:], atol=1e-10)


def _explicit_obs_gptq(W, H, perm, bits, group_size, static=None):
    """The column loop by the route of [derivation] sections 4 and 6: for
    each column, the full OBS update (eq. (22)) with the current inverse
    Hessian of the free coordinates, then its rank-1 downdate (eq. (26)).
    No Cholesky factor and no blocking; dynamic groups fitted on the current
    working row at each group start.  ``static`` = (scales, zeros) [m, n_g]
    on the original column layout: original column k uses group k // g."""
    Wp = np.array(W[:, perm], dtype=np.float64)
    m, d = Wp.shape
    G = np.linalg.inv(H)
    codes = np.zeros((m, d), dtype=np.int64)
    scales = []
    if group_size == -1:
        sc, z = orc.fit_grid(W, bits)
    for j in range(d):
        if static is not None:
            k = perm[j]
            sc, z = static[0][:, k // group_size], static[1][:, k // group_size]
        elif group_size > 0 and j % group_size == 0:
            sc, z = orc.fit_grid(Wp[:, j:j + group_size], bits)
            scales.append(sc)
        c, q, _ = orc.encode(Wp[:, j], sc, z, bits)
        codes[:, j] = c
        for r in range(m):
            delta, _ = orc.obs_update(G, 0, Wp[r, j] - q[r])
            Wp[r, j:] += delta
        G = orc.downdate(G, 0)
    return codes, scales


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("group_size", [-1, 3, 8])
def test_full_loop_equals_explicit_obs_with_downdates(seed, group_size):
    """The Cholesky/lazy-block loop equals the explicit OBS + downdate route
    column for column, including dynamic-group refits and act-order."""
    rng = np.random.default_rng(100 + seed)
    m, d, n = 6, 16, 60
    W, Xt = rand_layer(rng, m, d, n)
    Xt[:, 5] *= 4.0
    S = orc.hessian_sum(Xt)
    act = bool(seed % 2)
    b = 8 if group_size != 3 else 3
    res = orc.gptq_layer(W, S, n, bits=3, group_size=group_size, blocksize=b,
                         act_order=act)
    H, perm, _, damp = orc.prepare(S, n, 0.01, act)
    codes, scales = _explicit_obs_gptq(W, H + damp * np.eye(d), perm, 3,
                                       group_size)
    np.testing.assert_array_equal(res.codes_perm, codes)
    if group_size > 0:
        np.testing.assert_allclose(res.scales, np.stack(scales, axis=1))


@pytest.mark.parametrize("seed", range(4))
def test_R_tail_identity(seed):
    """eq. (40): (R[j:, j:])^T R[j:, j:] = (H_lambda[j:, j:])^-1 for all j."""
    rng = np.random.default_rng(seed)
    W, Xt = rand_layer(rng, 4, 12, 40)
    S = orc.hessian_sum(Xt)
    H, perm, dead, damp = orc.prepare(S, 40, 0.01, bool(seed % 2))
    R, damp = orc.factor(H, damp)
    Hl = H + damp * np.eye(12)
    assert np.allclose(np.tril(R, -1), 0.0)
    assert np.all(np.diag(R) > 0)
    for j in range(12):
        T = R[j:, j:]
        np.testing.assert_allclose(T.T @ T, np.linalg.inv(Hl[j:, j:]),
                                   rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("group_size", [-1, 4])
def test_loss_accounting_identity(seed, group_size):
    """[derivation] section 5 and eq. (67): with lambda = 0 and full-rank H
    the sum of the per-step increments rho^2 / (2 R_jj^2) equals the true
    layer error (1/N)||(W - W_hat) X||_F^2, for any grid choices."""
    rng = np.random.default_rng(seed)
    W, Xt = rand_layer(rng, 6, 10, 64)
    S = orc.hessian_sum(Xt)
    res = orc.gptq_layer(W, S, 64, bits=3, group_size=group_size,
                         blocksize=4, percdamp=0.0, damp_override=0.0,
                         act_order=bool(seed % 2))
    X = Xt.T
    err_direct = np.sum(((W - res.w_hat) @ X) ** 2) / 64
    assert abs(orc.layer_error(W, res.w_hat, S, 64) - err_direct) < 1e-12
    assert abs(orc.proxy_loss(res.rho_perm, res.R) - err_direct) < 1e-9 * max(1, err_direct)


def test_gptq_beats_rtn_on_average():
    """GPTQ should lower the layer error versus RTN on the same row grid."""
    rng = np.random.default_rng(7)
    wins = 0
    for _ in range(8):
        W, Xt = rand_layer(rng, 16, 24, 96, rank=8)
        S = orc.hessian_sum(Xt)
        res = orc.gptq_layer(W, S, 96, bits=3, group_size=-1, blocksize=8)
        sc, z = orc.fit_grid(W, 3)
        _, q = orc.rtn(W, sc, z, 3)
        wins += orc.layer_error(W, res.w_hat, S, 96) < orc.layer_error(W, q, S, 96)
    assert wins >= 7


@pytest.mark.parametrize("group_size", [-1, 8])
@pytest.mark.parametrize("act_order", [False, True])
def test_diagonal_H_reduces_to_rtn(group_size, act_order):
    """[derivation] 4.5 check and 11.2 remark: with a diagonal H there is no
    compensation, so GPTQ codes are the round-to-nearest codes."""
    rng = np.random.default_rng(3)
    m, d = 7, 24
    W = rng.standard_normal((m, d))
    S = np.diag(rng.uniform(0.5, 3.0, d))
    res = orc.gptq_layer(W, S, 10, bits=4, group_size=group_size,
                         blocksize=8, act_order=act_order)
    assert np.allclose(res.R - np.diag(np.diag(res.R)), 0.0)
    if group_size == -1:
        sc, z = orc.fit_grid(W, 4)
        c, _ = orc.rtn(W, sc, z, 4)
    else:
        # groups are formed in processing order
        Wp = W[:, res.perm]
        c = np.zeros((m, d), dtype=np.int64)
        for j0 in range(0, d, group_size):
            sc, z = orc.fit_grid(Wp[:, j0:j0 + group_size], 4)
            cc, _ = orc.rtn(Wp[:, j0:j0 + group_size], sc, z, 4)
            c[:, res.perm[j0:j0 + group_size]] = cc
    np.testing.assert_array_equal(res.codes, c)


@pytest.mark.parametrize("bits,group_size", [(4, -1), (3, 8), (2, 16)])
def test_blocksize_invariance(bits, group_size):
    """[derivation] eq. (49): lazy batching changes only the grouping of the
    same updates -- blocksize 1 and 128 give the same codes."""
    rng = np.random.default_rng(11)
    W, Xt = rand_layer(rng, 12, 48, 200, rank=12)
    S = orc.hessian_sum(Xt)
    outs = [orc.gptq_layer(W, S, 200, bits=bits, group_size=group_size,
                           blocksize=b) for b in (1, 16, 128)]
    for o in outs[1:]:
        np.testing.assert_array_equal(o.codes, outs[0].codes)
        np.testing.assert_allclose(o.w_hat, outs[0].w_hat, atol=1e-9)


def test_act_order_is_a_consistent_permutation():
    """eq. (34)/(35): act-order on (W, X) equals natural-order GPTQ on the
    pre-permuted layer (W Pi^T, Pi X), mapped back; W'X' = WX."""
    rng = np.random.default_rng(5)
    m, d, n = 9, 20, 80
    W, Xt = rand_layer(rng, m, d, n)
    Xt[:, 3] *= 6.0
    S = orc.hessian_sum(Xt)
    res = orc.gptq_layer(W, S, n, bits=3, group_size=4, blocksize=8,
                         act_order=True)
    perm = res.perm
    assert np.all(np.diff(np.diag(S)[perm]) <= 0)
    Wp, Xp = W[:, perm], Xt[:, perm]
    np.testing.assert_allclose(Wp @ Xp.T, W @ Xt.T, atol=1e-12)
    res2 = orc.gptq_layer(Wp, orc.hessian_sum(Xp), n, bits=3, group_size=4,
                          blocksize=8, act_order=False)
    np.testing.assert_array_equal(res.codes[:, perm], res2.codes)
    np.testing.assert_allclose(res.scales, res2.scales)
    np.testing.assert_array_equal(res.g_idx[perm], np.arange(d) // 4)


def test_act_order_stable_ties():
    """Equal diagonals keep their original relative order."""
    S = np.diag([1.0, 3.0, 1.0, 3.0, 2.0])
    _, perm, _, _ = orc.prepare(S, 2, 0.01, True)
    np.testing.assert_array_equal(perm, [1, 3, 4, 0, 2])


def test_column_lands_on_q_and_nonnegative_increments():
    """[derivation] 4.5 verifications: after its own update column j equals
    q exactly; every increment is >= 0; a diagonal G moves nothing else."""
    rng = np.random.default_rng(2)
    H = rand_spd(rng, 8)
    R, _ = orc.factor(H, 0.0)
    W = rng.standard_normal((3, 8))
    scale = np.full(3, 0.2, dtype=np.float32)
    zero = np.full(3, 8)
    Wc = W.copy()
    for j in range(8):
        _, q, _ = orc.encode(Wc[:, j], scale, zero, 4)
        eta = (Wc[:, j] - q) / R[j, j]
        Wc[:, j:] -= eta[:, None] * R[j, j:][None, :]
        np.testing.assert_allclose(Wc[:, j], q, atol=1e-12)
        assert np.all(eta ** 2 / 2 >= 0)
    delta, _ = orc.obs_update(np.diag([1.0, 2.0, 3.0]), 1, 0.5)
    np.testing.assert_allclose(delta, [0.0, -0.5, 0.0])


def test_gptq_not_globally_optimal_but_bounded_by_brute_force():
    """[derivation] section 4 opening remark: GPTQ is greedy, so exhaustive
    search over the same fixed grid gives a loss <= the GPTQ loss."""
    rng = np.random.default_rng(9)
    for _ in range(5):
        W, Xt = rand_layer(rng, 1, 4, 16)
        S = orc.hessian_sum(Xt)
        grid = (np.array([0.02], dtype=np.float32), np.array([2]))
        res = orc.gptq_layer(W, S, 16, bits=2, group_size=-1, blocksize=2,
                             percdamp=0.0, damp_override=0.0, fixed_grid=grid)
        levels = float(grid[0][0]) * (np.arange(4) - 2)   # same float32 step
        best = min(orc.layer_error(W, np.array([cand]), S, 16)
                   for cand in itertools.product(levels, repeat=4))
        assert best <= orc.layer_error(W, res.w_hat, S, 16) * (1 + 1e-12)


def test_dead_features():
    """[derivation] section 10: never-seen inputs get H_jj = 1 and their
    working weights are zeroed, so they quantize to the code of 0."""
    rng = np.random.default_rng(4)
    W, Xt = rand_layer(rng, 5, 16, 40)
    Xt[:, [2, 9]] = 0.0
    S = orc.hessian_sum(Xt)
    res = orc.gptq_layer(W, S, 40, bits=4, group_size=-1, blocksize=4)
    np.testing.assert_array_equal(np.nonzero(res.dead)[0], [2, 9])
    np.testing.assert_allclose(res.w_hat[:, [2, 9]], 0.0, atol=1e-12)
    np.testing.assert_array_equal(res.codes[:, 2], res.zeros[:, 0])


def test_retry_on_indefinite_and_not_spd():
    H = np.array([[1.0, 2.5], [2.5, 1.0]])          # eigenvalues 3.5, -1.5
    R, damp = orc.factor(H, 1e-3)
    assert damp > 1.0 and abs(damp - 10.0) < 1e-9    # 1e-3 * 10^4
    np.testing.assert_allclose(R.T @ R, np.linalg.inv(H + damp * np.eye(2)))
    with pytest.raises(orc.NotSPDError):
        orc.factor(np.array([[-1e6]]), 1e-3)


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_pack_roundtrip_and_bit_positions(bits):
    """The packing layout (our reading): code c of column k occupies stream
    bits [k*b, (k+1)*b), LSB first, in little-endian uint32 words."""
    rng = np.random.default_rng(bits)
    d = 37
    codes = rng.integers(0, 2 ** bits, size=(3, d))
    packed = orc.pack_codes(codes, bits)
    assert packed.shape == (3, -(-d * bits // 32))
    np.testing.assert_array_equal(orc.unpack_codes(packed, d, bits), codes)
    # brute force: rebuild every word bit by bit from a Python integer
    for r in range(3):
        big = 0
        for k in range(d):
            big |= int(codes[r, k]) << (k * bits)
        for w in range(packed.shape[1]):
            assert int(packed[r, w]) == (big >> (32 * w)) & 0xFFFFFFFF


def test_pack_hand_example():
    """4-bit codes 1..8 fill one word as 0x87654321; 3-bit codes cross a word
    boundary at column 10 (bits 30..32)."""
    c4 = np.arange(1, 9)[None, :]
    assert int(orc.pack_codes(c4, 4)[0, 0]) == 0x87654321
    c3 = np.zeros((1, 12), dtype=np.int64)
    c3[0, 10] = 0b111
    p = orc.pack_codes(c3, 3)
    assert int(p[0, 0]) == 0xC0000000 and int(p[0, 1]) == 0x1


def test_fit_grid_conventions():
    w = np.array([[-1.0, 0.5, 2.0], [0.0, 0.0, 0.0], [1.0, 2.0, 3.0]])
    sc, z = orc.fit_grid(w, 4)
    assert sc.dtype == np.float32
    np.testing.assert_allclose(sc, [3.0 / 15, 2.0 / 15, 3.0 / 15], rtol=1e-7)
    # row 2: float32(2/15) rounds up, so 1/Delta = 7.4999995 -> 7 (an exact
    # 7.5 would round to the even 8): the decision is taken in float32
    np.testing.assert_array_equal(z, [5, 7, 0])
    c, q, _ = orc.encode(w[2], np.full(3, sc[2]), np.full(3, z[2]), 4)
    np.testing.assert_array_equal(c, [5, 10, 15])


def test_group_layout_rule():
    assert orc.check_group_layout(256, 128, 128)
    assert orc.check_group_layout(256, 64, 128)
    assert orc.check_group_layout(512, 256, 128)
    assert orc.check_group_layout(300, 300, 128)
    assert not orc.check_group_layout(512, 96, 128)
    assert orc.check_group_layout(100, 96, 128)     # second group is the tail
    with pytest.raises(ValueError):
        orc.quantize_columns(np.zeros((1, 512)), np.eye(512), 4, 96, 128)


def test_ragged_shapes_run():
    rng = np.random.default_rng(1)
    W, Xt = rand_layer(rng, 3, 37, 50)
    S = orc.hessian_sum(Xt)
    res = orc.gptq_layer(W, S, 50, bits=3, group_size=-1, blocksize=16)
    assert res.codes.shape == (3, 37) and res.packed.shape == (3, 4)
    assert res.codes.min() >= 0 and res.codes.max() <= 7


# ----------------------------------------------------------------------------
# Quantizer variants: symmetric (signed) grid, ternary, static groups
# ----------------------------------------------------------------------------

def test_symmetric_grid_hand_example():
    """Symmetric 4-bit grid on [-0.33, 0.7, 0.12, -0.2]: a = 0.7, 15 levels
    -7..7, Delta = a / 7 = 0.1, z = 7; w / Delta = -3.3, 7, 1.2, -2 round
    to the signed codes -3, 7, 1, -2 (unsigned 4, 14, 8, 5)."""
    w = np.array([[-0.33, 0.7, 0.12, -0.2]])
    sc, z = orc.fit_grid(w, 4, symmetric=True)
    assert abs(float(sc[0]) - 0.1) < 1e-7 and int(z[0]) == 7
    c, q, _ = orc.encode(w[0], sc[0], z[0], 4, orc.grid_maxq(4, True))
    np.testing.assert_array_equal(c - 7, [-3, 7, 1, -2])
    np.testing.assert_allclose(q, [-0.3, 0.7, 0.1, -0.2], atol=1e-7)


def test_ternary_grid_hand_example():
    """[teardown] "extreme quantization": the ternary grid {-1, 0, +1} Delta
    is the symmetric 2-bit grid.  A group of 8 with max |w| = 0.3 gets
    Delta = 0.3; w / Delta rounds to -1, 0 or +1 only."""
    w = np.array([[0.3, -0.1, 0.16, -0.2, 0.05, -0.3, 0.0, 0.29]])
    sc, z = orc.fit_grid(w, 2, symmetric=True)
    assert abs(float(sc[0]) - 0.3) < 1e-7 and int(z[0]) == 1
    c, q, _ = orc.encode(w[0], sc[0], z[0], 2, orc.grid_maxq(2, True))
    np.testing.assert_array_equal(c - 1, [1, 0, 1, -1, 0, -1, 0, 1])
    assert set(np.round(q / 0.3, 6)) <= {-1.0, 0.0, 1.0}


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
def test_symmetric_grid_is_odd_and_exact_at_extremes(bits):
    """The symmetric grid maps -w to -q(w) (away from ties), represents 0
    and +-max|w| exactly, and rounds every w in range within Delta / 2."""
    rng = np.random.default_rng(bits)
    w = rng.standard_normal((5, 33))
    w[2] = 0.0
    sc, z = orc.fit_grid(w, bits, symmetric=True)
    mq = orc.grid_maxq(bits, True)
    assert np.all(z == 2 ** (bits - 1) - 1)
    for r in range(5):
        c, q, v = orc.encode(w[r], sc[r], z[r], bits, mq)
        cn, qn, _ = orc.encode(-w[r], sc[r], z[r], bits, mq)
        far = np.abs(v - np.floor(v) - 0.5) > 1e-6
        np.testing.assert_allclose(qn[far], -q[far], atol=0)
        assert np.all(np.abs(q - w[r]) <= sc[r] / 2 * (1 + 1e-6))
        if r != 2:
            a = np.max(np.abs(w[r]))
            k = int(np.argmax(np.abs(w[r])))
            assert abs(abs(q[k]) - a) <= 1e-6 * a
        c0, q0, _ = orc.encode(np.zeros(1), sc[r], z[r], bits, mq)
        assert q0[0] == 0.0


def test_symmetric_layer_codes_are_signed_two_complement():
    rng = np.random.default_rng(8)
    W, Xt = rand_layer(rng, 6, 20, 60)
    S = orc.hessian_sum(Xt)
    res = orc.gptq_layer(W, S, 60, bits=3, group_size=4, blocksize=8,
                         symmetric=True)
    signed = res.codes - 3
    assert signed.min() >= -3 and signed.max() <= 3
    unpacked = orc.unpack_codes(res.packed, 20, 3)
    np.testing.assert_array_equal(np.where(unpacked >= 4, unpacked - 8, unpacked),
                                  signed)
    np.testing.assert_allclose(res.w_hat,
                               res.scales[np.arange(6)[:, None], res.g_idx[None, :]]
                               * signed, atol=1e-12)


@pytest.mark.parametrize("act_order", [False, True])
def test_static_groups_diagonal_H_is_rtn_on_original_groups(act_order):
    """Static groups are fitted on the original contiguous columns, so with
    a diagonal H (no compensation) the codes are the group-wise RTN codes
    of the original layout whatever the processing order, and group_id is
    the trivial k // g ([derivation] 8.3)."""
    rng = np.random.default_rng(21)
    m, d, g = 5, 24, 8
    W = rng.standard_normal((m, d))
    S = np.diag(rng.uniform(0.5, 3.0, d))
    res = orc.gptq_layer(W, S, 10, bits=3, group_size=g, blocksize=8,
                         act_order=act_order, static_groups=True)
    np.testing.assert_array_equal(res.g_idx, np.arange(d) // g)
    for G in range(d // g):
        sc, z = orc.fit_grid(W[:, G * g:(G + 1) * g], 3)
        c, _ = orc.rtn(W[:, G * g:(G + 1) * g], sc, z, 3)
        np.testing.assert_array_equal(res.codes[:, G * g:(G + 1) * g], c)
        np.testing.assert_array_equal(res.scales[:, G], sc)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("symmetric", [False, True])
def test_static_groups_equal_explicit_obs(seed, symmetric):
    """With act-order, static groups (grid of processing position j =
    group floor(pi_j / g) of the original layout) through the Cholesky /
    lazy-block loop equal the explicit OBS + downdate route."""
    rng = np.random.default_rng(300 + seed)
    m, d, n, g = 6, 16, 60, 4
    W, Xt = rand_layer(rng, m, d, n)
    Xt[:, 7] *= 5.0
    S = orc.hessian_sum(Xt)
    res = orc.gptq_layer(W, S, n, bits=3, group_size=g, blocksize=3,
                         act_order=True, static_groups=True, symmetric=symmetric)
    H, perm, _, damp = orc.prepare(S, n, 0.01, True)
    assert not np.array_equal(perm, np.arange(d))
    grids = orc.static_group_grids(W, 3, g, symmetric)
    np.testing.assert_array_equal(res.scales, grids[0])
    codes = _explicit_static(W, H + damp * np.eye(d), perm, 3, g, grids,
                             orc.grid_maxq(3, symmetric))
    np.testing.assert_array_equal(res.codes_perm, codes)


def _explicit_static(W, H, perm, bits, g, grids, maxq):
    Wp = np.array(W[:, perm], dtype=np.float64)
    m, d = Wp.shape
    G = np.linalg.inv(H)
    codes = np.zeros((m, d), dtype=np.int64)
    for j in range(d):
        k = perm[j]
        c, q, _ = orc.encode(Wp[:, j], grids[0][:, k // g], grids[1][:, k // g],
                             bits, maxq)
        codes[:, j] = c
        for r in range(m):
            delta, _ = orc.obs_update(G, 0, Wp[r, j] - q[r])
            Wp[r, j:] += delta
        G = orc.downdate(G, 0)
    return codes


def test_static_groups_any_blocksize():
    """Static grids are fixed in advance, so no (g, blocksize) rule applies
    and every blocksize gives the same codes."""
    rng = np.random.default_rng(31)
    W, Xt = rand_layer(rng, 7, 40, 120, rank=10)
    S = orc.hessian_sum(Xt)
    outs = [orc.gptq_layer(W, S, 120, bits=4, group_size=12, blocksize=b,
                           static_groups=True, act_order=True) for b in (1, 7, 128)]
    for o in outs[1:]:
        np.testing.assert_array_equal(o.codes, outs[0].codes)


@pytest.mark.parametrize("group_size,act_order", [(-1, False), (8, True)])
def test_dequantize_stored_format_equals_loop_values(group_size, act_order):
    """Dequantizing the stored format (packed codes, scales, zeros, group
    ids) gives back the values the column loop quantized to -- for dynamic
    groups under act-order, static groups and the signed symmetric grid."""
    rng = np.random.default_rng(17)
    W, Xt = rand_layer(rng, 9, 40, 150)
    Xt[:, 11] *= 7.0
    S = orc.hessian_sum(Xt)
    for kw in (dict(), dict(static_groups=True), dict(symmetric=True)):
        res = orc.gptq_layer(W, S, 150, bits=3, group_size=group_size, blocksize=8,
                             act_order=act_order, **kw)
        zeros = np.zeros_like(res.zeros) if res.signed else res.zeros
        Wd = orc.dequantize(res.packed, res.scales, zeros, res.g_idx, 40, 3,
                            signed=res.signed)
        np.testing.assert_allclose(Wd, res.w_hat, atol=1e-15)
        x = rng.standard_normal((5, 40))
        np.testing.assert_allclose(
            orc.dequant_matmul(x, res.packed, res.scales, zeros, res.g_idx, 3,
                               signed=res.signed), x @ res.w_hat.T, atol=1e-12)


def test_bf16_round_against_torch():
    """bf16_round agrees with torch's float32 -> bfloat16 conversion (round
    to nearest even) on values exactly representable in float32."""
    import torch
    rng = np.random.default_rng(23)
    v = np.concatenate([rng.standard_normal(5000) * 10 ** rng.uniform(-6, 6, 5000),
                        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5, 0.0, 255.5]])
    v32 = v.astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(orc.bf16_round(v32.astype(np.float64)), ref)


def test_stack_layer_inputs_are_previous_outputs():
    """Layer-wise quantization: layer l+1's statistics come from layer l's
    quantized outputs; the first layer equals a lone gptq_layer call."""
    rng = np.random.default_rng(29)
    X0 = np.round(rng.standard_normal((300, 24)) * 2) / 2
    Ws = [0.05 * rng.standard_normal((16, 24)), 0.05 * rng.standard_normal((12, 16))]
    ps = [dict(bits=4, group_size=8, blocksize=8), dict(bits=3, group_size=-1, blocksize=4)]
    out, Xf = orc.gptq_stack(Ws, X0, ps, activation="relu")
    lone = orc.gptq_layer(Ws[0], orc.hessian_sum(X0), 300, **ps[0])
    np.testing.assert_array_equal(out[0]["res"].codes, lone.codes)
    X1 = orc.bf16_round(np.maximum(X0 @ lone.w_hat.T, 0.0))
    np.testing.assert_array_equal(out[1]["X"], X1)
    np.testing.assert_allclose(out[1]["S"], X1.T @ X1, rtol=1e-12)
    direct = np.sum(((Ws[1] - out[1]["res"].w_hat) @ X1.T) ** 2) / 300
    assert abs(out[1]["err"] - direct) <= 1e-12 * direct
    np.testing.assert_array_equal(
        Xf, orc.bf16_round(np.maximum(X1 @ out[1]["res"].w_hat.T, 0.0)))
