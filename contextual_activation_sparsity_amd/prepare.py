"""Offline preparation of the SVD predictor's inputs: factors and per-neuron thresholds.

This is set-up, not the decode path. It runs once per layer before serving, with torch
linear algebra on the host or the device, and hands svd_predict its bf16 factors and
fp32 thresholds. "SVD Contextual Sparsity Predictors for Fast LLM Inference" (abstract,
Figure 1): a low-rank SVD predictor with calibrated per-neuron thresholds, built
offline; Table 3 adds data whitening.
"""

from typing import Dict, Optional, Tuple

import torch


def _work_dtype(t: torch.Tensor) -> torch.dtype:
    return torch.float64 if t.device.type == "cpu" else torch.float32


def _decompose(w_gate: torch.Tensor, x_cal: Optional[torch.Tensor], ridge: float):
    """(U, s, Vh, S): the SVD of w_gate, or of w_gate S with S the Cholesky factor of the
    calibration tokens' second moment (S None without whitening)."""
    wd = _work_dtype(w_gate)
    W = w_gate.to(wd)
    if x_cal is None:
        U, s, Vh = torch.linalg.svd(W, full_matrices=False)
        return U, s, Vh, None
    X = x_cal.to(device=W.device, dtype=wd)
    if X.ndim != 2 or X.shape[1] != W.shape[1] or X.shape[0] < X.shape[1]:
        # with fewer tokens than d the second moment is singular: the ridge alone then
        # decides the factors, and in fp32 the Cholesky factorization can fail
        raise ValueError("whitening needs calibration tokens x_cal [n, d] with n >= d")
    C = X.T @ X / X.shape[0]
    C = C + ridge * torch.trace(C) / C.shape[0] * torch.eye(C.shape[0], dtype=wd, device=W.device)
    S = torch.linalg.cholesky(C)
    U, s, Vh = torch.linalg.svd(W @ S, full_matrices=False)
    return U, s, Vh, S


def _truncate(U, s, Vh, S, r: int, dtype: torch.dtype) -> Tuple[torch.Tensor, torch.Tensor]:
    if not (1 <= r <= s.numel()):
        raise ValueError("rank r must lie in [1, min(f, d)]")
    if S is None:
        q = Vh[:r]
    else:
        # q = V_r^T S^{-1}, i.e. S^T q^T = V_r
        q = torch.linalg.solve_triangular(S.T, Vh[:r].T, upper=True).T
    lf = U[:, :r] * s[:r]
    return q.to(dtype).contiguous(), lf.to(dtype).contiguous()


def svd_factors(w_gate: torch.Tensor, r: int, x_cal: Optional[torch.Tensor] = None, ridge: float = 1e-6,
                dtype: torch.dtype = torch.bfloat16) -> Tuple[torch.Tensor, torch.Tensor]:
    """Rank-r predictor factors q [r, d] and l [f, r] of the gate w_gate [f, d].

    Without calibration tokens: the truncated SVD w_gate = U diag(s) V^T, q = V_r^T,
    l = U_r diag(s_r) (the best rank-r approximation). With calibration tokens x_cal
    [n, d] (data whitening): the factors minimize the mean squared prediction error over
    those tokens. With the second moment C = x^T x / n = S S^T (Cholesky, plus a small
    ridge), take the truncated SVD of w_gate S and map it back: q = V_r^T S^{-1}.
    Whitening needs at least d calibration tokens.
    """
    if not (1 <= r <= min(w_gate.shape)):
        raise ValueError("rank r must lie in [1, min(f, d)]")
    return _truncate(*_decompose(w_gate, x_cal, ridge), r, dtype)


def svd_factors_ranks(w_gate: torch.Tensor, ranks, x_cal: Optional[torch.Tensor] = None, ridge: float = 1e-6,
                      dtype: torch.dtype = torch.bfloat16) -> Dict[int, Tuple[torch.Tensor, torch.Tensor]]:
    """svd_factors at several ranks from one decomposition: {r: (q, l)}."""
    ranks = [int(r) for r in ranks]
    if any(not (1 <= r <= min(w_gate.shape)) for r in ranks):
        raise ValueError("rank r must lie in [1, min(f, d)]")
    dec = _decompose(w_gate, x_cal, ridge)
    return {r: _truncate(*dec, r, dtype) for r in ranks}


def predictions(q: torch.Tensor, lf: torch.Tensor, x: torch.Tensor, b: Optional[torch.Tensor] = None) -> torch.Tensor:
    """p = l (q x) (+ b) for tokens x [n, d] (rows), in the working precision."""
    wd = _work_dtype(x)
    p = (x.to(wd) @ q.to(wd).T) @ lf.to(wd).T
    return p + b.to(wd) if b is not None else p


def calibrate_tau(p: torch.Tensor, g: torch.Tensor, s: float) -> torch.Tensor:
    """Per-neuron thresholds from calibration predictions p and true gates g ([n, f]).

    The pages say s sets the sparsity (Table 1) and that zero thresholding loses active
    neurons (Figure 2), without a formula. Rule used: per neuron, the mean prediction
    over tokens whose gate is inactive (m0) and over those where it is active (m1), and
    tau = (1 - s) m0 + s m1; 0 when either class is empty.
    """
    wd = _work_dtype(p)
    p = p.to(wd)
    on = (g > 0).to(wd)
    n_on, n_off = on.sum(0), (1 - on).sum(0)
    m_on = (p * on).sum(0) / n_on.clamp(min=1)
    m_off = (p * (1 - on)).sum(0) / n_off.clamp(min=1)
    tau = (1 - s) * m_off + s * m_on
    tau = torch.where((n_on > 0) & (n_off > 0), tau, torch.zeros_like(tau))
    return tau.to(torch.float32).contiguous()
