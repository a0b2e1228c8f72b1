"""The pins must catch plausible mistakes in the oracle.

Each case plants one mistake (a dropped term, a wrong sign, a wrong index or
operand, a transposed layout) in a copy of oracle/gdn_oracle.c, builds it on
the CPU, and checks that at least one pin fails.  Every mutant stays memory
safe (indices remain in bounds), so a mutant can only give wrong numbers.
"""
import functools
import os

import pytest

import oracle
from oracle import build as oracle_build
from oracle_pins import ALL_PINS, BWD_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")

H0_IDX = "P->h0[(((int64_t)n * P->Hv + j) * dk + i) * dv + c0 + c]"
HT_IDX = "P->ht[(((int64_t)n * P->Hv + j) * dk + i) * dv + c0 + c]"
UPD = "M[(int64_t)i * w + c] = a * M[(int64_t)i * w + c] + ki * delta[c];"

MUTANTS = {
    "prediction_not_decayed": ("delta[c] = b * ((double)vt[c] - a * y);",
                               "delta[c] = b * ((double)vt[c] - y);"),
    "beta_dropped": ("delta[c] = b * ((double)vt[c] - a * y);",
                     "delta[c] = ((double)vt[c] - a * y);"),
    "prediction_sign": ("delta[c] = b * ((double)vt[c] - a * y);",
                        "delta[c] = b * ((double)vt[c] + a * y);"),
    "state_not_decayed": (UPD, "M[(int64_t)i * w + c] = M[(int64_t)i * w + c] + ki * delta[c];"),
    "write_decayed_too": (UPD, "M[(int64_t)i * w + c] = a * (M[(int64_t)i * w + c] + ki * delta[c]);"),
    "output_reads_k": ("acc += M[(int64_t)i * w + c] * (double)qt[i];",
                       "acc += M[(int64_t)i * w + c] * (double)kt[i];"),
    "prediction_reads_q": ("y += M[(int64_t)i * w + c] * (double)kt[i];",
                           "y += M[(int64_t)i * w + c] * (double)qt[i];"),
    "grouped_heads_interleaved": ("const int32_t hk = j / G;", "const int32_t hk = j % P->Hqk;"),
    "decay_half_log": ("const double a = exp((double)P->g[p * P->Hv + j]);",
                       "const double a = exp(0.5 * (double)P->g[p * P->Hv + j]);"),
    "beta_complement": ("const double b = (double)P->beta[p * P->Hv + j];",
                        "const double b = 1.0 - (double)P->beta[p * P->Hv + j];"),
    "initial_state_ignored": ("P->h0 ? P->h0[", "0 ? P->h0["),
    "initial_state_transposed": (H0_IDX, "P->h0[(((int64_t)n * P->Hv + j) * dv + c0 + c) * dk + i]"),
    "final_state_transposed": (HT_IDX, "P->ht[(((int64_t)n * P->Hv + j) * dv + c0 + c) * dk + i]"),
    "scale_dropped": ("ot[c] = P->scale * acc;", "ot[c] = acc;"),
    "document_start_skipped": ("p0 = P->cu[n];", "p0 = P->cu[n] + (P->cu[n] < P->cu[n + 1]);"),
}


@functools.lru_cache(maxsize=None)
def _source():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = _source()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = oracle_build.build(str(path), str(tmp_path / f"lib{name}.so"))
    fwd = functools.partial(oracle.gdn_fwd, lib_path=lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(fwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the mutant {name}"


# Mistakes in the reverse mode; the forward pins never run it, so these must be
# caught by the reverse-mode pins (with the correct forward for the finite
# differences).
BWD_MUTANTS = {
    "bwd_dq_unscaled": ("dq[i] = P->scale * acc;", "dq[i] = acc;"),
    "bwd_dy_sign": ("acc2 += a * Mprev[(int64_t)i * dv + c] * (-b * W->dd[c]);",
                    "acc2 += a * Mprev[(int64_t)i * dv + c] * (b * W->dd[c]);"),
    "bwd_dk_write_term_dropped": ("dkk[i] = acc + acc2;", "dkk[i] = acc2;"),
    "bwd_dg_not_scaled_by_a": ("P->dg[row] = a * dga;", "P->dg[row] = dga;"),
    "bwd_state_grad_not_decayed": ("dM[e] = a * dP[e];", "dM[e] = dP[e];"),
    "bwd_dbeta_without_prediction": ("dbeta += dd * ((double)vt[c] - W->y[c]);",
                                     "dbeta += dd * (double)vt[c];"),
    "bwd_dv_missing_beta": ("dvv[c] = b * dd;", "dvv[c] = dd;"),
    "bwd_output_grad_previous_state": ("acc += Mt[(int64_t)i * dv + c] * (double)dot[c];",
                                       "acc += Mprev[(int64_t)i * dv + c] * (double)dot[c];"),
    "bwd_final_state_grad_ignored": ("dM[e] = P->dht ? P->dht[", "dM[e] = 0 ? P->dht["),
    "bwd_group_sum_first_head_only": ("for (int32_t gi = 0; gi < G; ++gi) {",
                                      "for (int32_t gi = 0; gi < 1; ++gi) {"),
    "bwd_dP_without_prediction_term": (
        "const double v_ = dM[(int64_t)i * dv + c] + (double)kt[i] * (-b * W->dd[c]);",
        "const double v_ = dM[(int64_t)i * dv + c];"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_pins_catch_mutant(name, tmp_path):
    old, new = BWD_MUTANTS[name]
    src = _source()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = oracle_build.build(str(path), str(tmp_path / f"lib{name}.so"))
    bwd = functools.partial(oracle.gdn_bwd, lib_path=lib)
    caught = []
    for pin in BWD_PINS:
        try:
            pin(oracle.gdn_fwd, bwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no reverse-mode pin catches the mutant {name}"


# Mistakes in the preparation and decode step (oracle/prep.py), planted in a
# copy of its source that is executed as a module of its own.
PREP_SRC = os.path.join(os.path.dirname(oracle.__file__), "prep.py")
PREP_MUTANTS = {
    "l2_sum_of_squares_not_rooted": ("n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))",
                                     "n = np.sum(x * x, axis=-1, keepdims=True)"),
    "l2_wrong_axis": ("n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))",
                      "n = np.sqrt(np.sum(x * x, axis=0, keepdims=True))"),
    "logsigmoid_negative_branch_sign": ("np.where(x >= 0.0, pos, x + pos)",
                                        "np.where(x >= 0.0, pos, x - pos)"),
    "logsigmoid_one_branch": ("np.where(x >= 0.0, pos, x + pos)", "pos"),
    "sigmoid_negative_branch": ("np.where(x >= 0.0, 1.0 / (1.0 + e), e / (1.0 + e))",
                                "np.where(x >= 0.0, 1.0 / (1.0 + e), 1.0 / (1.0 + e))"),
    "step_prediction_not_decayed": ("delta = beta[n, j] * (v[n, j] - a * y)",
                                    "delta = beta[n, j] * (v[n, j] - y)"),
    "step_state_not_decayed": ("M = a * M + np.outer(kv, delta)", "M = M + np.outer(kv, delta)"),
    "step_output_reads_k": ("o[n, j] = scale * (M.T @ qv)", "o[n, j] = scale * (M.T @ kv)"),
    "step_scale_dropped": ("o[n, j] = scale * (M.T @ qv)", "o[n, j] = (M.T @ qv)"),
    "step_grouped_heads_interleaved": ("kv, qv = k[n, j // G], q[n, j // G]",
                                       "kv, qv = k[n, j % Hqk], q[n, j % Hqk]"),
    "step_padding_reads_a_slot": ("cached = 0 <= s < S", "cached = s < S"),
    "step_gate_decay_not_log": ("g, beta = logsigmoid(g), sigmoid(beta)",
                                "g, beta = sigmoid(g), sigmoid(beta)"),
    "step_l2_keys_only": ("q, k = l2_normalize(q), l2_normalize(k)",
                          "q, k = q, l2_normalize(k)"),
    "l2_bwd_no_projection": ("return np.where(n > 0.0, (dy - proj * y) / safe, 0.0)",
                             "return np.where(n > 0.0, dy / safe, 0.0)"),
    "l2_bwd_not_divided_by_norm": ("return np.where(n > 0.0, (dy - proj * y) / safe, 0.0)",
                                   "return np.where(n > 0.0, dy - proj * y, 0.0)"),
    "l2_bwd_projects_on_raw_row": ("proj = np.sum(dy * y, axis=-1, keepdims=True)",
                                   "proj = np.sum(dy * x, axis=-1, keepdims=True)"),
    "logsigmoid_bwd_wrong_sign": ("np.asarray(dy, np.float64) * sigmoid(-np.asarray(x, np.float64))",
                                  "np.asarray(dy, np.float64) * sigmoid(np.asarray(x, np.float64))"),
    "sigmoid_bwd_one_factor": ("np.asarray(dy, np.float64) * sigmoid(x) * sigmoid(-x)",
                               "np.asarray(dy, np.float64) * sigmoid(x)"),
    "chain_gates_swapped": ("dg, dbeta = logsigmoid_bwd(g, dg), sigmoid_bwd(beta, dbeta)",
                            "dg, dbeta = sigmoid_bwd(g, dg), logsigmoid_bwd(beta, dbeta)"),
    "chain_keys_use_query_rows": ("dq, dk = l2_normalize_bwd(q, dq), l2_normalize_bwd(k, dk)",
                                  "dq, dk = l2_normalize_bwd(q, dq), l2_normalize_bwd(q, dk)"),
}


@pytest.mark.parametrize("name", sorted(PREP_MUTANTS))
def test_prep_pins_catch_mutant(name):
    import types
    from oracle_pins import PREP_BWD_PINS, PREP_PINS
    old, new = PREP_MUTANTS[name]
    with open(PREP_SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mod = types.ModuleType(f"prep_{name}")
    exec(compile(src.replace(old, new), f"prep_{name}.py", "exec"), mod.__dict__)
    caught = []
    for pin in PREP_PINS + PREP_BWD_PINS:
        try:
            pin(mod, oracle.gdn_fwd)
        except (AssertionError, IndexError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the mutant {name}"
