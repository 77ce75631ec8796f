"""CATS threshold calibration (float64).

TEST INFRASTRUCTURE: see the package docstring. Imports numpy only.

"CATS: Contextually-Aware Thresholding for Sparsity in Large Language Models" (abstract)
sets one threshold per layer so that a chosen fraction of activations (50% in the
abstract's headline) is zeroed. The reading used here: pool the scores
|SiLU(x Wg^T)| of every neuron over every calibration token of the layer and take the
K-th smallest, with K the rank that a target sparsity k names.
"""

import numpy as np

from .ffn import silu


def order_statistic_rank(k, N):
    """Rank K = floor(k N + 1/2) (1-based) of the threshold for sparsity k over N scores.

    K = 0 means "no neuron is cut" and K = N means "every neuron is cut". Rounding
    half up picks the nearest integer when k N is fractional; when k N is an integer
    K = k N, the count any order-statistic percentile definition gives.
    """
    if not (0.0 <= k <= 1.0):
        raise ValueError("sparsity k must lie in [0, 1]")
    return int(np.floor(np.float64(k) * N + 0.5))


def cats_scores(G):
    """CATS scores |SiLU(g)| of gates G (any shape, float64)."""
    return np.abs(silu(G))


def calibrate_cats(Wg, Xcal, k, b=None):
    """Threshold t for CATS sparsity k from calibration tokens Xcal [n, d].

    S = |SiLU(Xcal Wg^T (+ b))| ([n, f], float64), N = n f, K = order_statistic_rank.
    t is the K-th smallest element of S (1-based), so exactly K scores (all of them
    distinct) satisfy S <= t and are cut by the strict test |a| > t. K = 0 returns
    -1 (every score passes), K = N returns +inf (none passes).

    Returns (t as float64, t rounded to float32 by round-to-nearest-even, K, S).
    """
    Wg = np.asarray(Wg, dtype=np.float64)
    X = np.atleast_2d(np.asarray(Xcal, dtype=np.float64))
    G = X @ Wg.T
    if b is not None:
        G = G + np.asarray(b, dtype=np.float64)[None, :]
    S = cats_scores(G)
    N = S.size
    K = order_statistic_rank(k, N)
    if K == 0:
        t = -1.0
    elif K >= N:
        t = np.inf
    else:
        t = float(np.sort(S, axis=None)[K - 1])
    return t, np.float32(t), K, S
