"""Plants plausible mistakes in a copy of the oracle (on the CPU) and checks
that the pin suite catches every one of them.

Each mutation is a textual edit of oracle/gptq_ref.py's source, executed as a
fresh module; the pin and property tests are then re-run against it with the
module reference swapped.  A mutation that no test rejects would mean the
oracle is not pinned on that point.
"""

import inspect
import sys
import types

import pytest

import oracle.gptq_ref as ref
import test_oracle_pins as pins
import test_oracle_props as props

MUTATIONS = {
    # dropped term: no zero point in the encoder
    "encode_no_zero": ("c = np.clip(np.rint(v) + zero, 0, maxq)",
                       "c = np.clip(np.rint(v), 0, maxq)"),
    # wrong rounding
    "encode_floor": ("c = np.clip(np.rint(v) + zero, 0, maxq)",
                     "c = np.clip(np.floor(v) + zero, 0, maxq)"),
    # multiply instead of divide by R_jj
    "eta_times_rjj": ("eta = rho / R[j, j]", "eta = rho * R[j, j]"),
    # sign error in the in-block update
    "inblock_sign": ("W[:, j:i2] -= eta[:, None] * R[j, j:i2][None, :]",
                     "W[:, j:i2] += eta[:, None] * R[j, j:i2][None, :]"),
    # in-block update reading a column of R instead of its row
    "inblock_R_column": ("W[:, j:i2] -= eta[:, None] * R[j, j:i2][None, :]",
                         "W[:, j:i2] -= eta[:, None] * R[j:i2, j][None, :]"),
    # lazy tail update dropped
    "no_lazy_tail": ("W[:, i2:] -= E @ R[i:i2, i2:]", "pass"),
    # transposed operand in the lazy tail
    "lazy_transposed": ("W[:, i2:] -= E @ R[i:i2, i2:]",
                        "W[:, i2:] -= E @ R[i2:, i:i2].T"),
    # lower factor instead of upper
    "R_lower": ("R = np.linalg.cholesky(G).T", "R = np.linalg.cholesky(G)"),
    # Cholesky of H instead of H^-1
    "R_of_H": ("R = np.linalg.cholesky(G).T", "R = L.T"),
    # forgot the factor 2 of eq. (9)
    "hessian_no_2": ("return (2.0 / float(n)) *", "return (1.0 / float(n)) *"),
    # ascending act-order
    "act_order_ascending": ("perm = np.argsort(-np.diag(H), kind=\"stable\")",
                            "perm = np.argsort(np.diag(H), kind=\"stable\")"),
    # permutation applied to one side only
    "perm_one_side": ("H = H[np.ix_(perm, perm)]", "H = H"),
    # dead columns not zeroed
    "dead_not_zeroed": ("Wp[:, dead] = 0.0", "pass"),
    # wrong unpermute direction
    "unpermute_wrong": ("codes[:, perm] = out[\"codes\"]",
                        "codes[:, :] = out[\"codes\"][:, perm]"),
    # grid range not widened to include 0
    "grid_no_zero": ("lo = np.minimum(w.min(axis=1), 0.0).astype(np.float32)",
                     "lo = w.min(axis=1).astype(np.float32)"),
    # grid denominator off by one
    "grid_levels": ("maxq = np.float32(2 ** bits - 1)",
                    "maxq = np.float32(2 ** bits)"),
    # groups refitted on the original instead of the working weights
    "group_fit_wrong_cols": ("grp = W[:, j:min(j + group_size, d)]",
                             "grp = Wp[:, j:min(j + group_size, d)]"),
    # packing with the wrong bit order
    "pack_msb": ("stream[:, np.arange(d) * bits + k] = (codes >> k) & 1",
                 "stream[:, np.arange(d) * bits + (bits - 1 - k)] = (codes >> k) & 1"),
    # damping applied with the wrong sign
    "damp_sign": ("Hd = H + damp * eye", "Hd = H - damp * eye"),
    # damping relative to the sum / the largest diagonal entry, or none
    "damp_sum": ("damp = max(percdamp * float(np.mean(np.diag(H))), EPS_FLOOR)",
                 "damp = max(percdamp * float(np.sum(np.diag(H))), EPS_FLOOR)"),
    "damp_max": ("damp = max(percdamp * float(np.mean(np.diag(H))), EPS_FLOOR)",
                 "damp = max(percdamp * float(np.max(np.diag(H))), EPS_FLOOR)"),
    "damp_none": ("damp = max(percdamp * float(np.mean(np.diag(H))), EPS_FLOOR)",
                  "damp = EPS_FLOOR"),
    # wrong placeholder diagonal for never-seen features
    "dead_diag_2": ("H[idx, idx] = 1.0", "H[idx, idx] = 2.0"),
    # zero point floored instead of rounded
    "zero_floor": ("zero = np.rint((-lo) / scale).astype(np.float32)",
                   "zero = np.floor((-lo) / scale).astype(np.float32)"),
    # symmetric grid with 2^b levels (an off-centre zero point)
    "sym_levels": ("maxq = np.float32(grid_maxq(bits, True))",
                   "maxq = np.float32(2 ** bits - 1)"),
    # symmetric range taken from the positive side only
    "sym_one_sided": ("hi = np.maximum(-lo, hi)", "hi = hi"),
    # static group of position j taken in processing order, not floor(pi_j/g)
    "static_gpos_processing": ("static_grid=(sg[0], sg[1], perm // group_size)",
                               "static_grid=(sg[0], sg[1], np.arange(d) // group_size)"),
    # static group ids permuted like dynamic ones
    "static_gidx_permuted": ("        g_idx = np.arange(d) // group_size\n",
                             "        g_idx[perm] = np.arange(d) // group_size\n"),
    # dequantization ignoring the group id of each column
    "dequant_no_gidx": ("return scales[rows, g_idx[None, :]] * (codes - zeros[rows, g_idx[None, :]])",
                        "return scales[rows, :1] * (codes - zeros[rows, :1])"),
    # signed codes not sign-extended
    "dequant_no_sign": ("codes = np.where(codes >= 2 ** (bits - 1), codes - 2 ** bits, codes)",
                        "pass"),
    # next layer fed by the unquantized layer's outputs
    "stack_float_propagation": ("Y = dequant_matmul(X, res.packed, res.scales, zeros, res.g_idx,",
                                "Y = X @ W.T if True else dequant_matmul(X, res.packed, res.scales, zeros, res.g_idx,"),
    # activation skipped between layers
    "stack_no_activation": ("X = bf16_round(activate(Y, activation))", "X = bf16_round(Y)"),
    # symmetric codes stored unsigned
    "signed_codes_unsigned": ("return np.mod(res.codes - z, 2 ** bits)",
                              "return res.codes"),
}


def mutated_module(name):
    old, new = MUTATIONS[name]
    src = inspect.getsource(ref)
    assert src.count(old) == 1, f"mutation anchor not unique: {name}"
    mod = types.ModuleType(f"oracle_mut_{name}")
    sys.modules[mod.__name__] = mod          # dataclasses look the module up
    try:
        exec(compile(src.replace(old, new), f"<{name}>", "exec"), mod.__dict__)
    finally:
        del sys.modules[mod.__name__]
    return mod


def run_battery(mod):
    """Return the number of pin/property tests that fail against ``mod``."""
    failures = 0
    saved = (pins.orc, props.orc)
    pins.orc = props.orc = mod
    try:
        cases = []
        for m in (pins, props):
            for name, fn in inspect.getmembers(m, inspect.isfunction):
                if not name.startswith("test_"):
                    continue
                params = inspect.signature(fn).parameters
                if not params:
                    cases.append((fn, {}))
                elif set(params) == {"seed"}:
                    cases += [(fn, {"seed": s}) for s in range(2)]
                elif set(params) == {"bits"}:
                    cases += [(fn, {"bits": b}) for b in (3, 4)]
                elif set(params) == {"seed", "group_size"}:
                    cases += [(fn, {"seed": 1, "group_size": g}) for g in (-1, 4)]
                elif set(params) == {"group_size", "act_order"}:
                    cases += [(fn, {"group_size": g, "act_order": a})
                              for g in (-1, 8) for a in (False, True)]
                elif set(params) == {"bits", "group_size"}:
                    cases += [(fn, {"bits": 3, "group_size": 8})]
                elif set(params) == {"act_order"}:
                    cases += [(fn, {"act_order": a}) for a in (False, True)]
                elif set(params) == {"seed", "symmetric"}:
                    cases += [(fn, {"seed": 0, "symmetric": sy}) for sy in (False, True)]
                else:
                    raise AssertionError(f"battery cannot call {name}{tuple(params)}")
        for fn, kw in cases:
            try:
                fn(**kw)
            except KeyboardInterrupt:
                raise
            except BaseException:   # noqa: BLE001 - any failure counts,
                failures += 1       # pytest.fail / pytest.raises' Failed too
    finally:
        pins.orc, props.orc = saved
    return failures


def test_unmutated_oracle_passes_battery():
    assert run_battery(ref) == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    assert run_battery(mutated_module(name)) > 0, f"mutation {name} not caught"
