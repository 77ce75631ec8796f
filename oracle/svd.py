"""SVD sparsity predictor and the ReGLU sequential pipeline (float64).

TEST INFRASTRUCTURE: see the package docstring. Imports numpy only.

Source: "SVD Contextual Sparsity Predictors for Fast LLM Inference" -- abstract (a
training-free predictor from a truncated SVD of the gate projection, a threshold
calibration algorithm, ReGLU FFNs), Figure 1 (offline stage builds low-rank predictors
with per-neuron thresholds; at inference the predictor precedes each FFN block),
Figure 2 (zero thresholding of the predictor loses truly active neurons), Figure 3
(neurons with positive predictor values are treated as active; gate and up run one
after the other), Table 1 (the hyperparameter s sets the sparsity).
"""

import numpy as np

from .ffn import gate_up, relu


def svd_factors(Wg, r):
    """Rank-r truncated SVD of the gate projection Wg [f, d].

    Wg = U diag(sigma) V^T; the predictor keeps the r largest singular triplets and
    stores them as Q = V_r^T [r, d] and L = U_r diag(sigma_r) [f, r], so that
    L Q is the best rank-r approximation of Wg (Eckart-Young). The abstract's
    "truncation-aware" SVD and data whitening are not specified on the page; with
    inputs of identity covariance whitening is the identity, so the plain truncated
    SVD is the reading used here.
    """
    Wg = np.asarray(Wg, dtype=np.float64)
    if not (1 <= r <= min(Wg.shape)):
        raise ValueError("rank r must lie in [1, min(f, d)]")
    U, sig, Vt = np.linalg.svd(Wg, full_matrices=False)
    Q = Vt[:r, :].copy()
    L = U[:, :r] * sig[None, :r]
    return Q, L


def svd_factors_whitened(Wg, Xcal, r, ridge=1e-6):
    """Rank-r predictor of Wg fitted to the inputs it will see (data whitening).

    The pages list data whitening as a step that improves the predictor (Table 3,
    "+ Data whitening") without a formula. Reading used here: minimize the mean squared
    prediction error over the calibration tokens, E ||(Wg - L Q) x||^2, which is
    ||(Wg - L Q) S||_F^2 for the input second moment C = X^T X / n = S S^T (Cholesky;
    a ridge of `ridge` times the mean diagonal keeps C positive definite). Its minimizer
    is the truncated SVD of the whitened gate Wg S = U diag(sigma) V^T mapped back:
    L = U_r diag(sigma_r), Q = V_r^T S^{-1}. With C = I this is svd_factors.
    """
    Wg = np.asarray(Wg, dtype=np.float64)
    X = np.asarray(Xcal, dtype=np.float64)
    if not (1 <= r <= min(Wg.shape)):
        raise ValueError("rank r must lie in [1, min(f, d)]")
    C = X.T @ X / X.shape[0]
    C = C + ridge * np.trace(C) / C.shape[0] * np.eye(C.shape[0])
    S = np.linalg.cholesky(C)
    U, sig, Vt = np.linalg.svd(Wg @ S, full_matrices=False)
    L = U[:, :r] * sig[None, :r]
    Q = np.linalg.solve(S.T, Vt[:r, :].T).T  # V_r^T S^{-1}
    return Q, L


def svd_predict(Q, L, x, b=None):
    """Predicted gate p = L (Q x) (+ b) of one token (float64).

    Q x is the token projected on the top-r right singular vectors, L maps it back to
    one prediction per neuron. The predictor includes the gate bias because it
    predicts the biased gate whose sign decides ReLU activity.
    """
    z = np.asarray(Q, dtype=np.float64) @ np.asarray(x, dtype=np.float64)
    p = np.asarray(L, dtype=np.float64) @ z
    if b is not None:
        p = p + np.asarray(b, dtype=np.float64)
    return p


def svd_candidates(p, tau):
    """Candidate set {i : p_i > tau_i} (strict): neurons predicted active.

    With tau = 0 this is Figure 3's rule (positive predictor value means active).
    """
    return np.asarray(p, dtype=np.float64) > np.asarray(tau, dtype=np.float64)


def calibrate_tau(P, G, s):
    """Per-neuron predictor thresholds from calibration predictions.

    P, G: [n, f] predicted and true (biased) gates of n calibration tokens. The page
    says per-neuron thresholds fix the false negatives of zero thresholding (Figure 2)
    and that s implicitly sets the sparsity (Table 1) but gives no rule. Reading used
    here (parity unpinned against the page): split each neuron's calibration tokens
    by the sign of the true gate, take the mean prediction m+ over tokens with g > 0
    and m- over the rest, and interpolate, tau_i = (1 - s) m-_i + s m+_i. A neuron
    with an empty class keeps the zero threshold. tau rises with s because m+ > m-
    for a useful predictor, so the candidate set shrinks as s grows.
    """
    P = np.atleast_2d(np.asarray(P, dtype=np.float64))
    G = np.atleast_2d(np.asarray(G, dtype=np.float64))
    pos = G > 0.0
    n_pos = pos.sum(axis=0)
    n_neg = (~pos).sum(axis=0)
    tau = np.zeros(P.shape[1], dtype=np.float64)
    ok = (n_pos > 0) & (n_neg > 0)
    m_pos = np.where(pos, P, 0.0).sum(axis=0)[ok] / n_pos[ok]
    m_neg = np.where(~pos, P, 0.0).sum(axis=0)[ok] / n_neg[ok]
    tau[ok] = (1.0 - s) * m_neg + s * m_pos
    return tau


def reglu_sequential(Wg, Wu, Dt, x, cand, b=None):
    """ReGLU FFN of one token through the sequential pipeline of Figure 3.

    The gate is evaluated on the candidate rows only; the up projection only where
    ReLU(gate) > 0 there; the down projection over the same rows:
        active = cand and (g > 0),   y = sum_{i in active} g_i u_i Dt[i].
    Because ReLU already zeroes g <= 0, this equals the dense ReGLU FFN masked by
    cand. Returns (active mask [f], gate g [f], y [d]).
    """
    g, u = gate_up(Wg, Wu, x, b)
    c = np.asarray(cand, dtype=bool)
    active = c & (g > 0.0)
    h = np.where(active, relu(g) * u, 0.0)
    return active, g, np.asarray(Dt, dtype=np.float64).T @ h
