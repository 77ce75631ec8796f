"""Dense and masked gated FFN, the CATS mask, batches and the dense chunk (float64).

TEST INFRASTRUCTURE: see the package docstring. Imports numpy only.

Notation. Hidden size d, intermediate size f. Weights are row-major [f, d], one row per
neuron: ``Wg`` (gate), ``Wu`` (up) and ``Dt`` (the down projection stored transposed,
so row i holds neuron i's d output weights). For a token x in R^d:

    g = Wg x (+ b)       gate, one score per neuron
    u = Wu x             up projection
    a = act(g)           SiLU for SwiGLU / CATS, ReLU for ReGLU
    h = m * a * u        m = the 0/1 activity mask
    y = sum_i h_i Dt[i]  the FFN output

The method's result is this masked FFN exactly: sparsity enters only through m, there
is no approximation inside the active set. So the oracle is "dense FFN, then mask".
"""

import numpy as np


def bf16_to_f64(bits):
    """Decode bfloat16 bit patterns exactly.

    A bfloat16 value is the upper half of an IEEE-754 binary32 word, so shifting the
    16-bit pattern left by 16 gives the binary32 value, which float64 holds exactly.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def silu(g):
    """SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g)), in float64.

    The gated activation of the SwiGLU FFNs that CATS sparsifies ("CATS:
    Contextually-Aware Thresholding for Sparsity in Large Language Models", abstract).
    For g below about -709 exp(-g) overflows to inf and the quotient is -0.0, the
    correctly rounded limit.
    """
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def relu(g):
    """ReLU(g) = max(g, 0): the gate activation of the ReGLU FFNs that the SVD
    predictor targets ("SVD Contextual Sparsity Predictors for Fast LLM Inference",
    abstract)."""
    return np.maximum(np.asarray(g, dtype=np.float64), 0.0)


def activation(act):
    """'silu' or 'relu' -> the elementwise function."""
    if act == "silu":
        return silu
    if act == "relu":
        return relu
    raise ValueError(f"unknown activation {act!r}")


def gate_up(Wg, Wu, x, b=None):
    """Gate and up projections of one token: g = Wg x (+ b), u = Wu x (float64)."""
    Wg = np.asarray(Wg, dtype=np.float64)
    Wu = np.asarray(Wu, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    g = Wg @ x
    if b is not None:
        g = g + np.asarray(b, dtype=np.float64)
    u = Wu @ x
    return g, u


def dense_ffn(Wg, Wu, Dt, x, act="silu", b=None):
    """The full (dense) gated FFN of one token, y = sum_i act(g_i) u_i Dt[i].

    This is what the full model computes and what the Sirius verification pass
    reproduces ("SIRIUS: Contexual Sparisty with Correction for Efficient LLMs",
    Approach: sparse and full model share the weights).
    """
    g, u = gate_up(Wg, Wu, x, b)
    h = activation(act)(g) * u
    return np.asarray(Dt, dtype=np.float64).T @ h


def masked_ffn(Wg, Wu, Dt, x, mask, act="silu", b=None):
    """The FFN of one token restricted to the neurons where ``mask`` is true.

    y = sum_i m_i act(g_i) u_i Dt[i]. Only rows of Wu and Dt with m_i = 1 contribute,
    which is what lets a sparse executor read only those rows ("SVD Contextual
    Sparsity Predictors for Fast LLM Inference", abstract: conditional computation).
    """
    g, u = gate_up(Wg, Wu, x, b)
    m = np.asarray(mask, dtype=bool)
    h = np.where(m, activation(act)(g) * u, 0.0)
    return np.asarray(Dt, dtype=np.float64).T @ h


def cats_mask(a, t):
    """CATS activity mask: neuron i is active iff |a_i| > t (strict).

    The CATS abstract names a thresholding activation whose threshold is set per
    layer; the reading used here is a hard threshold on the magnitude of the SiLU
    output, kept unchanged where it passes and zeroed where it does not. Equality
    counts as inactive. t is the float32 threshold the library is given, widened.
    """
    return np.abs(np.asarray(a, dtype=np.float64)) > np.float64(t)


def cats_decode(Wg, Wu, Dt, X, t, act="silu", b=None, mask=None):
    """One CATS decode step for a batch of tokens X [B, d] (B >= 1).

    Per token b: scores a_b = act(g_b); mask m_b = |a_b| > t unless ``mask`` [B, f]
    is given, in which case it is used as is; y_b = masked FFN on m_b. Each token
    keeps its own mask even when a batch executor reads the union of the rows.
    Returns (masks [B, f] bool, scores [B, f], Y [B, d]).
    """
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    masks, scores, ys = [], [], []
    for j in range(X.shape[0]):
        g, _ = gate_up(Wg, Wu, X[j], b)
        a = activation(act)(g)
        m = cats_mask(a, t) if mask is None else np.asarray(mask[j], dtype=bool)
        masks.append(m)
        scores.append(a)
        ys.append(masked_ffn(Wg, Wu, Dt, X[j], m, act, b))
    return np.array(masks), np.array(scores), np.array(ys)


def union_mask(masks):
    """Rows a batch executor must read: the union over tokens of their masks."""
    return np.any(np.asarray(masks, dtype=bool), axis=0)


def dense_chunk(Wg, Wu, Dt, X, act="silu", b=None):
    """Dense FFN over a chunk of n tokens, Y[j] = dense_ffn(X[j]).

    Sirius has the full model verify a chunk of tokens produced by the sparse model in
    one parallel pass; its reported accepted advance lengths are out of 16 ("SIRIUS:
    Contexual Sparisty with Correction for Efficient LLMs", Approach and Key results),
    so chunks hold at most 16 tokens. At FFN level the pass is the dense FFN of each
    token of the chunk.
    """
    X = np.atleast_2d(np.asarray(X, dtype=np.float64))
    return np.array([dense_ffn(Wg, Wu, Dt, X[j], act, b) for j in range(X.shape[0])])


def within_threshold_band(score, t, rel=1e-3, abs_floor=0.0):
    """True where a score sits so close to its threshold that float32 and float64
    evaluation may legitimately decide differently: |score - t| <= rel*|t| + abs_floor.

    Used by the parity tests to excuse mask mismatches; everything outside the band
    must agree exactly.
    """
    s = np.asarray(score, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    return np.abs(s - t) <= rel * np.abs(t) + abs_floor
