"""The predictor-quality measures of contextual_activation_sparsity_amd.diagnostics
(torch) against the oracle's (numpy float64) on the CPU."""

import numpy as np
import torch

import oracle
from contextual_activation_sparsity_amd import diagnostics as dg


def test_roc_auc_matches_oracle():
    g = np.random.default_rng(40)
    for n, levels in ((50, 4), (3000, 1000), (20000, None)):
        sc = g.integers(0, levels, size=n).astype(np.float64) if levels else g.standard_normal(n)
        lab = g.random(n) < 0.3
        lab[0], lab[1] = True, False
        a = dg.roc_auc(torch.from_numpy(sc), torch.from_numpy(lab))
        assert abs(a - oracle.roc_auc(sc, lab)) <= 1e-12
        # float32 scores, as the library writes them
        s32 = sc.astype(np.float32)
        assert abs(dg.roc_auc(torch.from_numpy(s32), torch.from_numpy(lab)) - oracle.roc_auc(s32, lab)) <= 1e-12


def test_recall_and_masks_from_lists():
    g = np.random.default_rng(41)
    f = 37
    act = g.random((5, f)) < 0.3
    act[:, 0] = True
    idx = np.full((5, f), -1, np.int32)
    cnt = np.zeros(5, np.int32)
    cand = np.zeros((5, f), bool)
    for j in range(5):
        rows = g.permutation(f)[: g.integers(0, f)]
        idx[j, : rows.size] = rows
        cnt[j] = rows.size
        cand[j, rows] = True
    m = dg.masks_from_lists(torch.from_numpy(idx), torch.from_numpy(cnt), f)
    assert np.array_equal(m.numpy(), cand)
    assert abs(dg.recall(m, torch.from_numpy(act)) - oracle.recall(cand, act)) <= 1e-15
