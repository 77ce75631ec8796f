"""The Sirius correction schedule at the level of one FFN layer group (float64).

TEST INFRASTRUCTURE: see the package docstring. Imports numpy and this package only.

"SIRIUS: Contexual Sparisty with Correction for Efficient LLMs" (Approach; Key results):
the sparse model produces a chunk of tokens, and the full model, which shares the
weights, verifies the whole chunk in one parallel pass. The page reports the cost as an
effective density (0.807 on GSM8K with an accepted advance length of 15.37 of 16) and
the quality gap as accuracy; it gives neither formula.

Without a language model there is no token to accept or roll back. What an FFN layer
group can show is (i) the bytes each generated token costs once the verification is
counted, and (ii) how far the sparse layer outputs sit from the full ones on the same
inputs. The readings:

* One period is ``period`` sparse decode steps, each token through every layer of the
  group, then one dense pass of the same ``period`` tokens per layer (the verification
  chunk). The dense pass reads each weight row once for the whole chunk.
* Effective density = (weight bytes of the period) / (accepted tokens x dense bytes of
  one token) = (period * rho_sparse + rho_verify) / aal, where rho is a step's weight
  bytes relative to one dense token's and aal the accepted advance length. With every
  token accepted, aal = period.
* Divergence of a token at a layer = ||y_sparse - y_dense||_2 / ||y_dense||_2, the
  relative L2 distance between the sparse and the full layer output on the same input.
"""

import numpy as np

from .ffn import cats_decode, dense_chunk


def effective_density(rho_sparse, period, aal, rho_verify=1.0):
    """Weight bytes per accepted token over those of one dense token (reading above).

    rho_sparse: bytes of one sparse step / bytes of one dense token (for CATS with a
    dense gate, (1 + 2 (1 - k)) / 3 at sparsity k); rho_verify: bytes of the verification
    pass / bytes of one dense token (1: each row is read once for the whole chunk).
    """
    period = int(period)
    aal = float(aal)
    if period < 1 or not (0.0 < aal <= period):
        raise ValueError("need period >= 1 and 0 < aal <= period")
    return (period * float(rho_sparse) + float(rho_verify)) / aal


def sparse_dense_divergence(y_sparse, y_dense):
    """Relative L2 distance per row: ||y_sparse - y_dense|| / ||y_dense||.

    Rows are the last axis. A zero dense row gives 0 if the sparse row is zero too, and
    inf otherwise.
    """
    ys = np.asarray(y_sparse, dtype=np.float64)
    yd = np.asarray(y_dense, dtype=np.float64)
    if ys.shape != yd.shape:
        raise ValueError("shapes differ")
    num = np.sqrt(np.sum((ys - yd) ** 2, axis=-1))
    den = np.sqrt(np.sum(yd ** 2, axis=-1))
    out = np.empty_like(num)
    zero = den == 0.0
    out[~zero] = num[~zero] / den[~zero]
    out[zero] = np.where(num[zero] == 0.0, 0.0, np.inf)
    return out


def period_outputs(layers, X, thresholds, act="silu"):
    """Outputs of one period over a layer group.

    layers: sequence of (Wg, Wu, Dt) per layer; X: [L, P, d], token j's input at layer
    l (each layer gets its own input, as in the decode stack); thresholds: the CATS
    threshold of each layer. Returns (Y_sparse [L, P, d], the CATS step of each token,
    and Y_dense [L, P, d], the verification chunk of each layer).
    """
    X = np.asarray(X, dtype=np.float64)
    if X.ndim != 3 or X.shape[0] != len(layers) or len(thresholds) != len(layers):
        raise ValueError("X must be [layers, tokens, d] with one threshold per layer")
    ys, yd = [], []
    for (Wg, Wu, Dt), Xl, t in zip(layers, X, thresholds):
        _, _, y = cats_decode(Wg, Wu, Dt, Xl, t, act=act)
        ys.append(y)
        yd.append(dense_chunk(Wg, Wu, Dt, Xl, act=act))
    return np.stack(ys), np.stack(yd)
