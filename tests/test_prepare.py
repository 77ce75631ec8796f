"""The offline SVD-predictor preparation (contextual_activation_sparsity_amd.prepare,
torch) against the oracle (numpy float64) on the CPU: the factors agree through their
product L Q (the factors themselves are unique only up to the sign of each singular
pair), whitened and not, and the per-neuron thresholds agree."""

import numpy as np
import torch

import oracle
from contextual_activation_sparsity_amd import inputs, prepare


def _case(seed=0, f=60, d=32):
    g = np.random.default_rng(seed)
    Wg = g.standard_normal((f, d)) * 0.2
    X = g.standard_normal((200, d)) @ np.diag(np.linspace(0.3, 2.0, d))
    return Wg, X


def test_plain_factors_match_oracle():
    Wg, _ = _case(1)
    for r in (1, 7, 32):
        q, lf = prepare.svd_factors(torch.from_numpy(Wg), r, dtype=torch.float64)
        Q, L = oracle.svd_factors(Wg, r)
        assert np.allclose(lf.numpy() @ q.numpy(), L @ Q, atol=1e-10)


def test_whitened_factors_match_oracle():
    Wg, X = _case(2)
    for r in (3, 16):
        q, lf = prepare.svd_factors(torch.from_numpy(Wg), r, x_cal=torch.from_numpy(X), dtype=torch.float64)
        Q, L = oracle.svd_factors_whitened(Wg, X, r)
        assert np.allclose(lf.numpy() @ q.numpy(), L @ Q, atol=1e-9)
        xs = X[:5]
        p = prepare.predictions(q, lf, torch.from_numpy(xs)).numpy()
        assert np.allclose(p, np.array([oracle.svd_predict(Q, L, x) for x in xs]), atol=1e-9)


def test_bf16_factors_are_rounded_products():
    Wg, _ = _case(3)
    q, lf = prepare.svd_factors(torch.from_numpy(Wg), 8)
    assert q.dtype == torch.bfloat16 and lf.dtype == torch.bfloat16
    assert q.shape == (8, Wg.shape[1]) and lf.shape == (Wg.shape[0], 8)
    q64, l64 = prepare.svd_factors(torch.from_numpy(Wg), 8, dtype=torch.float64)
    assert np.array_equal(q.view(torch.int16).numpy().view(np.uint16), inputs.f32_to_bf16_bits(q64.numpy().astype(np.float32)))


def test_tau_matches_oracle():
    g = np.random.default_rng(4)
    P = g.standard_normal((300, 50))
    G = P + 0.5 * g.standard_normal((300, 50))
    G[:, 7] = -1.0  # a neuron never active: zero threshold
    for s in (0.0, 0.3, 0.5, 1.0):
        t = prepare.calibrate_tau(torch.from_numpy(P), torch.from_numpy(G), s).numpy()
        to = oracle.calibrate_tau(P, G, s)
        assert np.allclose(t, to.astype(np.float32), rtol=1e-6, atol=1e-7)
        assert t[7] == 0.0


def test_whitening_rejects_too_few_tokens():
    Wg, X = _case(5)
    import pytest
    for bad in (X[:Wg.shape[1] - 1], X[:, :-1], X[0]):
        with pytest.raises(ValueError):
            prepare.svd_factors(torch.from_numpy(Wg), 4, x_cal=torch.from_numpy(bad))
    with pytest.raises(ValueError):
        prepare.svd_factors(torch.from_numpy(Wg), Wg.shape[1] + 1)


def test_factors_at_several_ranks_match_single_rank():
    Wg, X = _case(6)
    for xc in (None, torch.from_numpy(X)):
        multi = prepare.svd_factors_ranks(torch.from_numpy(Wg), (2, 9, 32), x_cal=xc, dtype=torch.float64)
        for r, (q, lf) in multi.items():
            q1, l1 = prepare.svd_factors(torch.from_numpy(Wg), r, x_cal=xc, dtype=torch.float64)
            assert np.allclose(lf.numpy() @ q.numpy(), l1.numpy() @ q1.numpy(), atol=1e-12)
