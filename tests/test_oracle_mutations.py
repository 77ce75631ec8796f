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
    "bf16_decode_shift": [(offn, "bf16_to_f64", _bf16_wrong_shift), (oracle, "bf16_to_f64", _bf16_wrong_shift)],
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
