"""Planted mistakes in the oracle (on the CPU) must each trip at least one pin.

Each mutation is a plausible slip -- a flipped sign, a transposed operand, a dropped
bias or absolute value, an off-by-one rank, a non-strict comparison -- patched into the
oracle for the duration of one check. The test passes when some pin fails on it, which
shows the pins are not blind to that mistake.
"""

import numpy as np
import pytest

import oracle
import oracle.calibrate as ocal
import oracle.diagnostics as odia
import oracle.ffn as offn
import oracle.sirius as osir
import oracle.svd as osvd
from tests import oracle_pins


def _silu_wrong_sign(g):
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(g))


def _gate_up_no_bias(Wg, Wu, x, b=None):
    return np.asarray(Wg, float) @ np.asarray(x, float), np.asarray(Wu, float) @ np.asarray(x, float)


def _cats_mask_ge(a, t):
    return np.abs(np.asarray(a, dtype=np.float64)) >= np.float64(t)


def _cats_mask_no_abs(a, t):
    return np.asarray(a, dtype=np.float64) > np.float64(t)


def _scores_no_abs(G):
    return offn.silu(G)


def _rank_off_by_one(k, N):
    return int(np.floor(k * N + 0.5)) + 1


def _svd_factors_no_sigma(Wg, r):
    U, sig, Vt = np.linalg.svd(np.asarray(Wg, float), full_matrices=False)
    return Vt[:r].copy(), U[:, :r].copy()


def _whitened_no_back_map(Wg, Xcal, r, ridge=1e-6):
    """Whitened SVD that forgets to map Q back through S^{-1}."""
    Wg = np.asarray(Wg, float)
    X = np.asarray(Xcal, float)
    C = X.T @ X / X.shape[0]
    C = C + ridge * np.trace(C) / C.shape[0] * np.eye(C.shape[0])
    S = np.linalg.cholesky(C)
    U, sig, Vt = np.linalg.svd(Wg @ S, full_matrices=False)
    return Vt[:r].copy(), U[:, :r] * sig[None, :r]


def _whitened_transposed_root(Wg, Xcal, r, ridge=1e-6):
    """Whitened SVD with the Cholesky factor on the wrong side (S^T instead of S)."""
    Wg = np.asarray(Wg, float)
    X = np.asarray(Xcal, float)
    C = X.T @ X / X.shape[0]
    C = C + ridge * np.trace(C) / C.shape[0] * np.eye(C.shape[0])
    S = np.linalg.cholesky(C).T
    U, sig, Vt = np.linalg.svd(Wg @ S, full_matrices=False)
    return np.linalg.solve(S.T, Vt[:r].T).T, U[:, :r] * sig[None, :r]


def _tau_swapped(P, G, s):
    return osvd.__dict__["_orig_calibrate_tau"](P, G, 1.0 - s)


def _dense_ffn_transposed(Wg, Wu, Dt, x, act="silu", b=None):
    g, u = offn.gate_up(Wg, Wu, x, b)
    h = offn.activation(act)(g) * u
    Dt = np.asarray(Dt, float)
    return (Dt @ h) if Dt.shape[1] == h.shape[0] else Dt.T @ h[::-1]


def _eff_density_no_verify(rho_sparse, period, aal, rho_verify=1.0):
    return float(rho_sparse) * int(period) / float(aal)


def _eff_density_per_period(rho_sparse, period, aal, rho_verify=1.0):
    return (int(period) * float(rho_sparse) + float(rho_verify)) / int(period)


def _divergence_sparse_norm(y_sparse, y_dense):
    ys, yd = np.asarray(y_sparse, float), np.asarray(y_dense, float)
    den = np.sqrt(np.sum(ys ** 2, axis=-1))
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.sqrt(np.sum((ys - yd) ** 2, axis=-1)) / den


def _auc_ties_win(scores, labels):
    from scipy import stats
    s, y = np.asarray(scores, float).ravel(), np.asarray(labels, bool).ravel()
    n1, n0 = int(y.sum()), int((~y).sum())
    return float((stats.rankdata(s, method="max")[y].sum() - n1 * (n1 + 1) / 2.0) / (n1 * n0))


def _auc_reference_swapped(scores, labels):
    from scipy import stats
    s, y = np.asarray(scores, float).ravel(), ~np.asarray(labels, bool).ravel()
    n1, n0 = int(y.sum()), int((~y).sum())
    return float((stats.rankdata(s)[y].sum() - n1 * (n1 + 1) / 2.0) / (n1 * n0))


def _recall_as_precision(candidates, active):
    c, a = np.asarray(candidates, bool), np.asarray(active, bool)
    return float(np.logical_and(c, a).sum() / c.sum())


def _bf16_wrong_shift(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)


def _band_rel_of_score(score, t, rel=1e-3, abs_floor=0.0):
    s, t = np.asarray(score, float), np.asarray(t, float)
    return np.abs(s - t) <= rel * np.abs(s) + abs_floor


def _band_strict(score, t, rel=1e-3, abs_floor=0.0):
    s, t = np.asarray(score, float), np.asarray(t, float)
    return np.abs(s - t) < rel * np.abs(t) + abs_floor


def _band_no_floor(score, t, rel=1e-3, abs_floor=0.0):
    s, t = np.asarray(score, float), np.asarray(t, float)
    return np.abs(s - t) <= rel * np.abs(t)


def _band_signed_t(score, t, rel=1e-3, abs_floor=0.0):
    s, t = np.asarray(score, float), np.asarray(t, float)
    return np.abs(s - t) <= rel * t + abs_floor


def _relu_leaky(g):
    g = np.asarray(g, dtype=np.float64)
    return np.where(g > 0.0, g, 0.01 * g)


def _union_as_intersection(masks):
    return np.all(np.asarray(masks, dtype=bool), axis=0)


def _masked_ffn_inverted(Wg, Wu, Dt, x, mask, act="silu", b=None):
    g, u = offn.gate_up(Wg, Wu, x, b)
    h = np.where(~np.asarray(mask, dtype=bool), offn.activation(act)(g) * u, 0.0)
    return np.asarray(Dt, dtype=np.float64).T @ h


def _cats_decode_first_mask(Wg, Wu, Dt, X, t, act="silu", b=None, mask=None):
    """Every token of the batch takes the first token's mask."""
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    masks, scores, ys = [], [], []
    for j in range(X.shape[0]):
        g, _ = offn.gate_up(Wg, Wu, X[j], b)
        a = offn.activation(act)(g)
        if j == 0:
            m0 = offn.cats_mask(a, t) if mask is None else np.asarray(mask[0], dtype=bool)
        masks.append(m0)
        scores.append(a)
        ys.append(offn.masked_ffn(Wg, Wu, Dt, X[j], m0, act, b))
    return np.array(masks), np.array(scores), np.array(ys)


def _dense_chunk_no_activation(Wg, Wu, Dt, X, act="silu", b=None):
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    out = []
    for j in range(X.shape[0]):
        g, u = offn.gate_up(Wg, Wu, X[j], b)
        out.append(np.asarray(Dt, dtype=np.float64).T @ (g * u))
    return np.array(out)


def _svd_predict_bias_subtracted(Q, L, x, b=None):
    p = np.asarray(L, dtype=np.float64) @ (np.asarray(Q, dtype=np.float64) @ np.asarray(x, dtype=np.float64))
    return p - np.asarray(b, dtype=np.float64) if b is not None else p


def _svd_candidates_ge(p, tau):
    return np.asarray(p, dtype=np.float64) >= np.asarray(tau, dtype=np.float64)


def _reglu_sequential_cand_ignored(Wg, Wu, Dt, x, cand, b=None):
    g, u = offn.gate_up(Wg, Wu, x, b)
    active = g > 0.0
    h = np.where(active, offn.relu(g) * u, 0.0)
    return active, g, np.asarray(Dt, dtype=np.float64).T @ h


def _fnr_as_one_minus_precision(candidates, active):
    c, a = np.asarray(candidates, dtype=bool), np.asarray(active, dtype=bool)
    return 1.0 - float((c & a).sum()) / max(int(c.sum()), 1)


def _period_dense_is_sparse(layers, X, thresholds, act="silu"):
    X = np.asarray(X, dtype=np.float64)
    ys = np.stack([offn.cats_decode(Wg, Wu, Dt, Xl, t, act=act)[2] for (Wg, Wu, Dt), Xl, t in zip(layers, X, thresholds)])
    return ys, ys.copy()


def _calibrate_zero_based(Wg, Xcal, k, b=None):
    """The K-th order statistic read with a 0-based index."""
    X = np.atleast_2d(np.asarray(Xcal, dtype=np.float64))
    G = X @ np.asarray(Wg, dtype=np.float64).T
    if b is not None:
        G = G + np.asarray(b, dtype=np.float64)[None, :]
    S = ocal.cats_scores(G)
    K = ocal.order_statistic_rank(k, S.size)
    t = -1.0 if K == 0 else np.inf if K >= S.size else float(np.sort(S, axis=None)[K])
    return t, np.float32(t), K, S


def _gate_up_wrong_matrix(Wg, Wu, x, b=None):
    """u taken from the gate matrix."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(Wg, dtype=np.float64) @ x
    if b is not None:
        g = g + np.asarray(b, dtype=np.float64)
    return g, np.asarray(Wg, dtype=np.float64) @ x


def _dense_ffn_act_on_u(Wg, Wu, Dt, x, act="silu", b=None):
    g, u = offn.gate_up(Wg, Wu, x, b)
    return np.asarray(Dt, dtype=np.float64).T @ (g * offn.activation(act)(u))


def _activation_swapped(act):
    if act == "silu":
        return offn.relu
    if act == "relu":
        return offn.silu
    raise ValueError(f"unknown activation {act!r}")


MUTATIONS = {
    "silu_sign": [(offn, "silu", _silu_wrong_sign)],
    "gate_bias_dropped": [(offn, "gate_up", _gate_up_no_bias), (osvd, "gate_up", _gate_up_no_bias)],
    "mask_non_strict": [(offn, "cats_mask", _cats_mask_ge)],
    "mask_no_abs": [(offn, "cats_mask", _cats_mask_no_abs)],
    "calibration_no_abs": [(ocal, "cats_scores", _scores_no_abs)],
    "rank_off_by_one": [(ocal, "order_statistic_rank", _rank_off_by_one)],
    "svd_sigma_dropped": [(osvd, "svd_factors", _svd_factors_no_sigma), (oracle, "svd_factors", _svd_factors_no_sigma)],
    "tau_classes_swapped": [(oracle, "calibrate_tau", _tau_swapped)],
    "whitened_no_back_map": [(osvd, "svd_factors_whitened", _whitened_no_back_map),
                             (oracle, "svd_factors_whitened", _whitened_no_back_map)],
    "whitened_transposed_root": [(osvd, "svd_factors_whitened", _whitened_transposed_root),
                                 (oracle, "svd_factors_whitened", _whitened_transposed_root)],
    "eff_density_no_verify": [(osir, "effective_density", _eff_density_no_verify),
                              (oracle, "effective_density", _eff_density_no_verify)],
    "eff_density_per_period": [(osir, "effective_density", _eff_density_per_period),
                               (oracle, "effective_density", _eff_density_per_period)],
    "divergence_sparse_norm": [(osir, "sparse_dense_divergence", _divergence_sparse_norm),
                               (oracle, "sparse_dense_divergence", _divergence_sparse_norm)],
    "auc_ties_count_as_wins": [(odia, "roc_auc", _auc_ties_win), (oracle, "roc_auc", _auc_ties_win)],
    "auc_classes_swapped": [(odia, "roc_auc", _auc_reference_swapped), (oracle, "roc_auc", _auc_reference_swapped)],
    "recall_as_precision": [(odia, "recall", _recall_as_precision), (oracle, "recall", _recall_as_precision)],
    "down_transposed": [(offn, "dense_ffn", _dense_ffn_transposed), (oracle, "dense_ffn", _dense_ffn_transposed)],
    "band_relative_to_score": [(offn, "within_threshold_band", _band_rel_of_score),
                               (oracle, "within_threshold_band", _band_rel_of_score)],
    "band_strict_edge": [(offn, "within_threshold_band", _band_strict),
                         (oracle, "within_threshold_band", _band_strict)],
    "band_floor_dropped": [(offn, "within_threshold_band", _band_no_floor),
                           (oracle, "within_threshold_band", _band_no_floor)],
    "band_signed_threshold": [(offn, "within_threshold_band", _band_signed_t),
                              (oracle, "within_threshold_band", _band_signed_t)],
    "bf16_decode_shift": [(offn, "bf16_to_f64", _bf16_wrong_shift), (oracle, "bf16_to_f64", _bf16_wrong_shift)],
    "relu_leaky": [(offn, "relu", _relu_leaky), (osvd, "relu", _relu_leaky), (oracle, "relu", _relu_leaky)],
    "union_as_intersection": [(offn, "union_mask", _union_as_intersection),
                              (oracle, "union_mask", _union_as_intersection)],
    "masked_ffn_mask_inverted": [(offn, "masked_ffn", _masked_ffn_inverted), (oracle, "masked_ffn", _masked_ffn_inverted)],
    "cats_decode_first_mask_for_all": [(offn, "cats_decode", _cats_decode_first_mask),
                                       (osir, "cats_decode", _cats_decode_first_mask),
                                       (oracle, "cats_decode", _cats_decode_first_mask)],
    "dense_chunk_no_activation": [(offn, "dense_chunk", _dense_chunk_no_activation),
                                  (osir, "dense_chunk", _dense_chunk_no_activation),
                                  (oracle, "dense_chunk", _dense_chunk_no_activation)],
    "svd_predict_bias_subtracted": [(osvd, "svd_predict", _svd_predict_bias_subtracted),
                                    (oracle, "svd_predict", _svd_predict_bias_subtracted)],
    "svd_candidates_non_strict": [(osvd, "svd_candidates", _svd_candidates_ge),
                                  (oracle, "svd_candidates", _svd_candidates_ge)],
    "reglu_sequential_cand_ignored": [(osvd, "reglu_sequential", _reglu_sequential_cand_ignored),
                                      (oracle, "reglu_sequential", _reglu_sequential_cand_ignored)],
    "fnr_as_one_minus_precision": [(odia, "false_negative_rate", _fnr_as_one_minus_precision),
                                   (oracle, "false_negative_rate", _fnr_as_one_minus_precision)],
    "calibration_zero_based_rank": [(ocal, "calibrate_cats", _calibrate_zero_based),
                                    (oracle, "calibrate_cats", _calibrate_zero_based)],
    "up_from_gate_matrix": [(offn, "gate_up", _gate_up_wrong_matrix), (osvd, "gate_up", _gate_up_wrong_matrix),
                            (oracle, "gate_up", _gate_up_wrong_matrix)],
    "activation_on_up": [(offn, "dense_ffn", _dense_ffn_act_on_u), (oracle, "dense_ffn", _dense_ffn_act_on_u)],
    "activations_swapped": [(offn, "activation", _activation_swapped), (oracle, "activation", _activation_swapped)],
    "period_dense_is_sparse": [(osir, "period_outputs", _period_dense_is_sparse),
                               (oracle, "period_outputs", _period_dense_is_sparse)],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    osvd.__dict__.setdefault("_orig_calibrate_tau", osvd.calibrate_tau)
    for mod, attr, fn in MUTATIONS[name]:
        monkeypatch.setattr(mod, attr, fn)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutation {name} passed every pin"
