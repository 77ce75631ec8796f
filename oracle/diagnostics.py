"""Quality of a sparsity predictor against the true activity (float64).

TEST INFRASTRUCTURE: see the package docstring. Imports numpy and scipy only.

"SVD Contextual Sparsity Predictors for Fast LLM Inference" rates its predictors by
layer-wise ROC AUC (Figures 4, 5 and 7: 1 is perfect separation, 0.5 random guessing;
the score reaches a plateau at a small rank) and shows that thresholding the prediction
at zero misses truly active neurons (Figure 2). The pages give no formula. Readings:

* Label of neuron i for token x: active iff the true gate is positive, g_i > 0 (ReGLU).
* Score: the predictor output p_i. A layer's ROC AUC pools all (token, neuron) pairs of
  the evaluation tokens: the probability that an active pair scores above an inactive
  one, ties counting one half (the Mann-Whitney form of the area under the ROC curve).
* Recall of a candidate set: active neurons that are candidates over all active
  neurons, pooled over tokens; the false-negative rate is 1 - recall.
"""

import numpy as np
from scipy import stats


def roc_auc(scores, labels):
    """Area under the ROC curve of ``scores`` for the boolean ``labels`` (same shape,
    pooled over all entries), by the rank-sum identity with average ranks for ties:
    AUC = (sum of the positives' ranks - n1 (n1 + 1) / 2) / (n1 n0).
    Needs at least one positive and one negative."""
    s = np.asarray(scores, dtype=np.float64).ravel()
    y = np.asarray(labels, dtype=bool).ravel()
    if s.shape != y.shape:
        raise ValueError("scores and labels differ in size")
    n1 = int(y.sum())
    n0 = y.size - n1
    if n1 == 0 or n0 == 0:
        raise ValueError("need both classes")
    ranks = stats.rankdata(s, method="average")
    return float((ranks[y].sum() - n1 * (n1 + 1) / 2.0) / (n1 * n0))


def recall(candidates, active):
    """Pooled recall |candidates and active| / |active| of boolean masks (same shape).
    Needs at least one active entry."""
    c = np.asarray(candidates, dtype=bool)
    a = np.asarray(active, dtype=bool)
    if c.shape != a.shape:
        raise ValueError("masks differ in shape")
    na = int(a.sum())
    if na == 0:
        raise ValueError("no active entry")
    return float(np.logical_and(c, a).sum() / na)


def false_negative_rate(candidates, active):
    """1 - recall: the share of truly active neurons the predictor drops."""
    return 1.0 - recall(candidates, active)
