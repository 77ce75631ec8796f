"""Predictor quality on the device: ROC AUC of predictor outputs against the true
activity, and the recall of candidate sets.

Analysis, not the decode path. "SVD Contextual Sparsity Predictors for Fast LLM
Inference" (Figures 2, 4, 5 and 7) rates predictors by layer-wise ROC AUC and shows
that a zero threshold loses truly active neurons. Here a neuron is active for a token
when its true gate is positive, its score is the predictor output, and a layer's AUC
pools all (token, neuron) pairs: the probability that an active pair scores above an
inactive one, ties counting one half.
"""

import torch


def roc_auc(scores: torch.Tensor, labels: torch.Tensor) -> float:
    """Area under the ROC curve of scores for boolean labels, pooled over all entries,
    from average ranks (ties share their mean rank). Works on any device, in float64."""
    s = scores.reshape(-1).to(torch.float64)
    y = labels.reshape(-1).to(torch.bool)
    if s.numel() != y.numel():
        raise ValueError("scores and labels differ in size")
    n1 = int(y.sum().item())
    n0 = y.numel() - n1
    if n1 == 0 or n0 == 0:
        raise ValueError("need both classes")
    _, inv, cnt = torch.unique(s, sorted=True, return_inverse=True, return_counts=True)
    end = torch.cumsum(cnt, 0).to(torch.float64)  # 1-based rank of each group's last entry
    avg = end - (cnt.to(torch.float64) - 1.0) / 2.0
    r1 = avg[inv][y].sum().item()
    return (r1 - n1 * (n1 + 1) / 2.0) / (float(n1) * float(n0))


def recall(candidates: torch.Tensor, active: torch.Tensor) -> float:
    """|candidates and active| / |active| over boolean masks of one shape, pooled."""
    c = candidates.to(torch.bool)
    a = active.to(torch.bool)
    if c.shape != a.shape:
        raise ValueError("masks differ in shape")
    na = int(a.sum().item())
    if na == 0:
        raise ValueError("no active entry")
    return int((c & a).sum().item()) / na


def masks_from_lists(idx: torch.Tensor, counts: torch.Tensor, f: int) -> torch.Tensor:
    """Boolean masks [n, f] from index lists [n, >= count] and their counts [n]: entry
    (j, idx[j, k]) is set for k < counts[j]."""
    n, width = idx.shape
    keep = torch.arange(width, device=idx.device)[None, :] < counts.reshape(-1, 1)
    m = torch.zeros((n, f), dtype=torch.bool, device=idx.device)
    rows = torch.arange(n, device=idx.device)[:, None].expand(n, width)
    m[rows[keep], idx[keep].long()] = True
    return m
