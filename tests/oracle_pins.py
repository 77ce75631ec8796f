"""Pins of the CPU oracle to values fixed by the source pages and by mathematics.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a value
that does not come from the oracle itself: a hand-worked golden fixture, a closed form,
a constructed input with a known answer, or an invariant of the definition. They are
collected by tests/test_oracle_pins.py and re-run against planted mistakes by
tests/test_oracle_mutations.py, which checks that each plausible mistake trips at least
one of them.
"""

import json
import math
import os

import numpy as np
from scipy import optimize, special, stats

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


W1E = float(special.lambertw(1.0 / math.e).real)  # W(1/e) = 0.27846...
G_STAR = -1.0 - W1E  # argmax of |SiLU| on the negative axis


def _closed_silu(v):
    return v / (1.0 + math.exp(-v))


# --------------------------------------------------------------------------- decode
def pin_bf16_patterns():
    fx = _load("bf16_patterns.json")
    expect = {
        "1": 1.0, "-3": -3.0, "1 + 2^-7": 1.0 + 2.0 ** -7, "3.140625": 3.140625,
        "2^-133": 2.0 ** -133, "2^-126": 2.0 ** -126,
        "(2 - 2^-7) * 2^127": (2.0 - 2.0 ** -7) * 2.0 ** 127,
        "-0": -0.0, "inf": math.inf, "-inf": -math.inf,
    }
    for case in fx["cases"]:
        got = float(oracle.bf16_to_f64(np.array([int(case["bits"], 16)], dtype=np.uint16))[0])
        want = expect[case["value"]]
        assert got == want, (case, got)
        assert math.copysign(1.0, got) == math.copysign(1.0, want), case


def pin_silu_closed_forms():
    for k in (2.0, 3.0, 5.0, 10.0):
        lk = math.log(k)
        assert abs(oracle.silu(lk) - lk * k / (k + 1.0)) <= 1e-15 * lk * k
        assert abs(oracle.silu(-lk) + lk / (k + 1.0)) <= 1e-15 * lk * k
    assert oracle.silu(0.0) == 0.0
    # |SiLU| peaks on the negative axis at g* = -1 - W(1/e) with value W(1/e).
    assert abs(abs(float(oracle.silu(G_STAR))) - W1E) <= 1e-15
    grid = np.linspace(-8.0, 0.0, 80001)
    vals = np.abs(oracle.silu(grid))
    assert vals.max() <= W1E + 1e-15
    assert abs(grid[int(np.argmax(vals))] - G_STAR) <= 2e-4
    # Large arguments: SiLU(g) -> g, SiLU(-g) -> -0.
    assert oracle.silu(60.0) == 60.0
    assert abs(float(oracle.silu(-800.0))) == 0.0


def pin_relu():
    assert list(oracle.relu([-2.0, -0.0, 0.0, 3.5])) == [0.0, 0.0, 0.0, 3.5]


# ------------------------------------------------------------------------ FFN + mask
def pin_reglu_golden():
    fx = _load("reglu_tiny.json")
    Wg, Wu, Dt = (np.array(fx[k], dtype=float) for k in ("Wg", "Wu", "Dt"))
    b, x = np.array(fx["b"], dtype=float), np.array(fx["x"], dtype=float)
    g, u = oracle.gate_up(Wg, Wu, x, b)
    assert np.array_equal(g, fx["g"])
    assert np.array_equal(oracle.dense_ffn(Wg, Wu, Dt, x, "relu", b), fx["y_dense"])
    for case in fx["cases"]:
        active, _, y = oracle.reglu_sequential(Wg, Wu, Dt, x, np.array(case["cand"], bool), b)
        assert np.array_equal(active.astype(int), case["active"]), case
        assert np.array_equal(y, case["y"]), (case, y)
        ym = oracle.masked_ffn(Wg, Wu, Dt, x, np.array(case["cand"], bool), "relu", b)
        assert np.array_equal(ym, case["y"]), case


def pin_cats_golden():
    fx = _load("cats_lnk.json")
    l3, l2 = math.log(3.0), math.log(2.0)
    x = np.array([l3, -l3, l2, -l2, 0.0])
    eye = np.eye(5)
    full = np.array([0.75 * l3 * l3, 0.25 * l3 * l3, (2.0 / 3.0) * l2 * l2, (1.0 / 3.0) * l2 * l2, 0.0])
    a_closed = np.array([0.75 * l3, -0.25 * l3, (2.0 / 3.0) * l2, -(1.0 / 3.0) * l2, 0.0])
    for case in fx["cases"]:
        masks, scores, Y = oracle.cats_decode(eye, eye, eye, x[None, :], case["t"])
        assert np.allclose(scores[0], a_closed, rtol=1e-15, atol=0), scores
        assert np.array_equal(masks[0].astype(int), case["mask"]), (case, masks)
        want = np.where(np.array(case["mask"], bool), full, 0.0)
        assert np.allclose(Y[0], want, rtol=1e-14, atol=0), (case, Y)


def pin_threshold_band():
    """Hand-worked band memberships (tests/golden/threshold_band.json): the edge
    |score - t| = rel |t| is inside, the half-width scales with |t| (not |score|), a
    zero threshold is widened only by the absolute floor, and per-token thresholds and
    per-neuron floors broadcast over a [tokens, neurons] score array."""
    fx = _load("threshold_band.json")
    for case in fx["cases"]:
        got = oracle.within_threshold_band(np.array(case["score"]), case["t"], case["rel"], case["abs_floor"])
        assert got.tolist() == case["in_band"], (case["what"], got.tolist())
    bc = fx["broadcast"]
    got = oracle.within_threshold_band(np.array(bc["score"]), np.array(bc["t"]), bc["rel"], np.array(bc["abs_floor"]))
    assert got.shape == (2, 3) and got.tolist() == bc["in_band"], got.tolist()
    # default rel is the contract's 1e-3
    assert oracle.within_threshold_band(1001.0, 1000.0) and not oracle.within_threshold_band(1001.0005, 1000.0)


def pin_asymmetric_shapes():
    """f != d with a non-symmetric Dt: y = sum_i h_i Dt[i] (rows of Dt are neurons)."""
    Wg = np.array([[1.0, 0.0, 0.0], [0.0, 2.0, 0.0]])  # f = 2, d = 3
    Wu = np.array([[1.0, 1.0, 1.0], [0.0, 0.0, 1.0]])
    Dt = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]])
    x = np.array([1.0, 1.0, 2.0])
    # g = [1, 2], relu = [1, 2], u = [4, 2], h = [4, 4], y = 4*[1,2,3] + 4*[4,5,6]
    y = oracle.dense_ffn(Wg, Wu, Dt, x, "relu")
    assert np.array_equal(y, [20.0, 28.0, 36.0]), y
    y0 = oracle.masked_ffn(Wg, Wu, Dt, x, np.array([False, True]), "relu")
    assert np.array_equal(y0, [16.0, 20.0, 24.0]), y0


def _rand_layer(seed, f, d, scale=0.3):
    g = np.random.default_rng(seed)
    return (g.standard_normal((f, d)) * scale, g.standard_normal((f, d)) * scale,
            g.standard_normal((f, d)) * scale, g.standard_normal(d), g.standard_normal(f) * 0.1)


def pin_relu_zero_threshold_is_dense():
    """ReLU with t = 0: masked FFN == dense FFN bit for bit (masked terms are exact 0)."""
    Wg, Wu, Dt, x, b = _rand_layer(1, 24, 16)
    m, _, Y = oracle.cats_decode(Wg, Wu, Dt, x[None], 0.0, act="relu", b=b)
    assert np.array_equal(Y[0], oracle.dense_ffn(Wg, Wu, Dt, x, "relu", b))
    g, _ = oracle.gate_up(Wg, Wu, x, b)
    assert np.array_equal(m[0], g > 0)


def pin_density_one_is_dense():
    """t = -1 (what calibration returns for k = 0): every neuron active, masked == dense."""
    Wg, Wu, Dt, x, _ = _rand_layer(2, 24, 16)
    m, _, Y = oracle.cats_decode(Wg, Wu, Dt, x[None], -1.0)
    assert m.all()
    assert np.allclose(Y[0], oracle.dense_ffn(Wg, Wu, Dt, x), rtol=1e-13, atol=1e-13)


def pin_mask_partition():
    """Linearity in the mask: y(m) + y(not m) == dense; an empty mask gives y = 0."""
    Wg, Wu, Dt, x, _ = _rand_layer(3, 40, 16)
    m = np.random.default_rng(4).random(40) < 0.4
    y1 = oracle.masked_ffn(Wg, Wu, Dt, x, m)
    y2 = oracle.masked_ffn(Wg, Wu, Dt, x, ~m)
    assert np.allclose(y1 + y2, oracle.dense_ffn(Wg, Wu, Dt, x), rtol=1e-12, atol=1e-12)
    assert np.array_equal(oracle.masked_ffn(Wg, Wu, Dt, x, np.zeros(40, bool)), np.zeros(16))


def pin_permutation():
    """Permuting neurons consistently permutes the mask and leaves y unchanged."""
    Wg, Wu, Dt, x, _ = _rand_layer(5, 32, 16)
    perm = np.random.default_rng(6).permutation(32)
    t = 0.2
    m, _, Y = oracle.cats_decode(Wg, Wu, Dt, x[None], t)
    mp, _, Yp = oracle.cats_decode(Wg[perm], Wu[perm], Dt[perm], x[None], t)
    assert np.array_equal(mp[0], m[0][perm])
    assert np.allclose(Yp, Y, rtol=1e-12, atol=1e-12)


def pin_brute_force_tiny():
    """Scalar loops, term by term, on a tiny random layer (d = 8, f = 16)."""
    Wg, Wu, Dt, x, b = _rand_layer(7, 16, 8, scale=0.7)
    t = 0.15
    want_y = [0.0] * 8
    want_m = []
    for i in range(16):
        gi = sum(Wg[i, j] * x[j] for j in range(8)) + b[i]
        ui = sum(Wu[i, j] * x[j] for j in range(8))
        ai = gi * (1.0 / (1.0 + math.exp(-gi)))
        on = abs(ai) > t
        want_m.append(on)
        if on:
            for j in range(8):
                want_y[j] += ai * ui * Dt[i, j]
    m, _, Y = oracle.cats_decode(Wg, Wu, Dt, x[None], t, b=b)
    assert list(m[0]) == want_m
    assert np.allclose(Y[0], want_y, rtol=1e-12, atol=1e-14)


def pin_batch_union():
    """Per-token masks in a batch: each token's result equals its single-token result;
    the union is exactly the rows some token needs."""
    Wg, Wu, Dt, _, _ = _rand_layer(8, 48, 16)
    X = np.random.default_rng(9).standard_normal((4, 16))
    t = 0.1
    M, _, Y = oracle.cats_decode(Wg, Wu, Dt, X, t)
    for j in range(4):
        mj, _, yj = oracle.cats_decode(Wg, Wu, Dt, X[j][None], t)
        assert np.array_equal(M[j], mj[0])
        assert np.array_equal(Y[j], yj[0])
    U = oracle.union_mask(M)
    assert np.array_equal(U, M[0] | M[1] | M[2] | M[3])


def pin_chunk_rows():
    """Rows of the dense chunk are per-token dense FFNs; the chunk is not a batch mix."""
    Wg, Wu, Dt, _, _ = _rand_layer(10, 24, 16)
    X = np.random.default_rng(11).standard_normal((16, 16))
    Y = oracle.dense_chunk(Wg, Wu, Dt, X)
    for j in (0, 7, 15):
        assert np.array_equal(Y[j], oracle.dense_ffn(Wg, Wu, Dt, X[j]))
    # Closed form with Wu = Wg = identity: y = Dt^T (SiLU(x) * x).
    eye = np.eye(16)
    Yi = oracle.dense_chunk(eye, eye, Dt[:16], X)
    want = np.array([Dt[:16].T @ (X[j] * X[j] / (1.0 + np.exp(-X[j]))) for j in range(16)])
    assert np.allclose(Yi, want, rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------------- calibration
def pin_calibration_known_order():
    fx = _load("calib_known.json")
    Xcal = np.array([[0.3, G_STAR, 0.5], [1.0, 2.0, 3.0]])
    named = {"SiLU(0.3)": _closed_silu(0.3), "W(1/e)": W1E, "SiLU(0.5)": _closed_silu(0.5),
             "SiLU(2)": _closed_silu(2.0), "-1": -1.0, "inf": math.inf}
    for case in fx["cases"]:
        t64, t32, K, _ = oracle.calibrate_cats(np.eye(3), Xcal, case["k"])
        assert K == case["K"], (case, K)
        want = named[case["t"]]
        if math.isinf(want):
            assert math.isinf(t64) and t64 > 0
        else:
            assert abs(t64 - want) <= 1e-15 * max(1.0, abs(want)), (case, t64, want)
            assert t32 == np.float32(want)


def pin_calibration_counts():
    """On distinct random scores exactly K are <= t and N - K pass the strict test."""
    g = np.random.default_rng(12)
    Wg = g.standard_normal((64, 32)) / math.sqrt(32)
    X = g.standard_normal((20, 32))
    for k in (0.1, 0.5, 0.7, 0.9, 0.333):
        t, _, K, S = oracle.calibrate_cats(Wg, X, k)
        assert K == math.floor(k * S.size + 0.5)
        assert int((S <= t).sum()) == K
        assert int((S > t).sum()) == S.size - K


def _gaussian_silu_quantile(k, sigma=1.0):
    """Closed-form k-quantile of |SiLU(sigma Z)|, Z ~ N(0,1), by root finding on
    F(t) = P(|SiLU(sigma Z)| <= t) written with the normal CDF."""
    f = lambda z: z / (1.0 + math.exp(-z))  # noqa: E731

    def cdf(t):
        zp = optimize.brentq(lambda z: f(z) - t, 0.0, 50.0)
        if t >= W1E:
            return stats.norm.cdf(zp / sigma)
        z1 = optimize.brentq(lambda z: -f(z) - t, -60.0, G_STAR)
        z2 = optimize.brentq(lambda z: -f(z) - t, G_STAR, 0.0)
        return stats.norm.cdf(z1 / sigma) + stats.norm.cdf(zp / sigma) - stats.norm.cdf(z2 / sigma)

    return optimize.brentq(lambda t: cdf(t) - k, 1e-9, 20.0)


def pin_calibration_gaussian():
    """Large iid sample: the calibrated threshold converges to the closed-form quantile."""
    x = np.random.default_rng(13).standard_normal((2000, 500))
    for k, tol in ((0.5, 4e-3), (0.7, 6e-3), (0.9, 1.5e-2)):
        t, _, _, _ = oracle.calibrate_cats(np.eye(500), x, k)
        want = _gaussian_silu_quantile(k)
        assert abs(t - want) <= tol, (k, t, want)
    assert abs(_gaussian_silu_quantile(0.5) - 0.254) < 2e-3


# ------------------------------------------------------------------------------- SVD
def _orthonormal(seed, n, k):
    q, r = np.linalg.qr(np.random.default_rng(seed).standard_normal((n, k)))
    return q * np.sign(np.diag(r))[None, :]


def pin_svd_constructed():
    """Wg = U diag(s) V^T with test-chosen s: L Q is the rank-r truncation, the
    residual is sum_{j>r} s_j^2 (Eckart-Young), Q has orthonormal rows, and an exactly
    rank-r matrix is reproduced."""
    f, d, r = 40, 24, 6
    U, V = _orthonormal(14, f, d), _orthonormal(15, d, d)
    s = np.sort(np.random.default_rng(16).uniform(0.1, 3.0, d))[::-1]
    Wg = (U * s) @ V.T
    Q, L = oracle.svd_factors(Wg, r)
    trunc = (U[:, :r] * s[:r]) @ V[:, :r].T
    assert np.allclose(L @ Q, trunc, rtol=0, atol=1e-12)
    res = np.linalg.norm(Wg - L @ Q) ** 2
    assert abs(res - (s[r:] ** 2).sum()) <= 1e-10 * (s ** 2).sum()
    assert np.allclose(Q @ Q.T, np.eye(r), atol=1e-12)
    assert Q.shape == (r, d) and L.shape == (f, r)
    low = (U[:, :r] * s[:r]) @ V[:, :r].T
    Q2, L2 = oracle.svd_factors(low, r)
    assert np.allclose(L2 @ Q2, low, atol=1e-12)


def pin_svd_predict_full_rank():
    """At full rank the predictor equals the biased gate, so with tau = 0 the candidate
    set is exactly {g > 0} (Figure 3's rule) and sequential ReGLU equals dense ReGLU."""
    Wg, Wu, Dt, x, b = _rand_layer(17, 20, 12)
    Q, L = oracle.svd_factors(Wg, 12)
    p = oracle.svd_predict(Q, L, x, b)
    g, _ = oracle.gate_up(Wg, Wu, x, b)
    assert np.allclose(p, g, atol=1e-12)
    cand = oracle.svd_candidates(p, np.zeros(20))
    assert np.array_equal(cand, g > 0)
    _, _, y = oracle.reglu_sequential(Wg, Wu, Dt, x, cand, b)
    assert np.allclose(y, oracle.dense_ffn(Wg, Wu, Dt, x, "relu", b), atol=1e-12)
    # rank-1 closed form: Wg = a c^T  ->  p = a (c . x) + b
    a, c = np.random.default_rng(18).standard_normal(20), np.random.default_rng(19).standard_normal(12)
    Q1, L1 = oracle.svd_factors(np.outer(a, c), 1)
    assert np.allclose(oracle.svd_predict(Q1, L1, x, b), a * (c @ x) + b, atol=1e-12)


def pin_svd_candidates_strict():
    """A neuron is a candidate only when its prediction is strictly above its threshold
    (SVDP Figure 3: a positive predictor value means active, and zero is not positive):
    hand-worked predictions at, just above and just below zero and per-neuron
    thresholds."""
    p = np.array([0.0, 1e-12, -1e-12, 0.5, 0.75, -0.25, 2.0])
    tau = np.array([0.0, 0.0, 0.0, 0.5, 0.5, -0.25, 2.5])
    assert oracle.svd_candidates(p, tau).tolist() == [False, True, False, False, True, False, False]


def pin_svd_whitened_identity():
    """Tokens whose second moment is exactly the identity (X = sqrt(n) times an
    orthonormal basis): the whitened predictor is the plain truncated SVD, L Q equal to
    the rank-r truncation of Wg."""
    f, d, r, n = 30, 12, 5, 48
    Wg = np.random.default_rng(20).standard_normal((f, d))
    X = np.sqrt(n) * _orthonormal(21, n, d)
    assert np.allclose(X.T @ X / n, np.eye(d), atol=1e-12)
    Qw, Lw = oracle.svd_factors_whitened(Wg, X, r, ridge=0.0)
    U, sg, Vt = np.linalg.svd(Wg, full_matrices=False)
    assert np.allclose(Lw @ Qw, (U[:, :r] * sg[:r]) @ Vt[:r], atol=1e-10)


def pin_svd_whitened_optimal():
    """Anisotropic tokens with a test-chosen covariance C = A A^T: over those tokens the
    whitened predictor's mean squared error is the tail energy sum_{j>r} s_j^2 of
    Wg C^{1/2} (any square root: the singular values do not depend on it), no larger
    than the plain SVD's error, and no rank-r perturbation of it does better."""
    f, d, r, n = 26, 10, 3, 400
    g = np.random.default_rng(22)
    Wg = g.standard_normal((f, d))
    A = g.standard_normal((d, d)) @ np.diag(np.linspace(0.1, 2.5, d))
    X = g.standard_normal((n, d)) @ A.T
    C = X.T @ X / n
    w, V = np.linalg.eigh(C)
    root = (V * np.sqrt(w)) @ V.T  # symmetric square root, not the oracle's Cholesky factor
    tail = (np.linalg.svd(Wg @ root, compute_uv=False)[r:] ** 2).sum()
    Qw, Lw = oracle.svd_factors_whitened(Wg, X, r, ridge=0.0)
    mse = lambda M: np.mean(np.sum((X @ (Wg - M).T) ** 2, axis=1))  # noqa: E731
    assert abs(mse(Lw @ Qw) - tail) <= 1e-9 * tail
    Qp, Lp = oracle.svd_factors(Wg, r)
    assert mse(Lw @ Qw) <= mse(Lp @ Qp) * (1 + 1e-12)
    for k in range(3):
        dl = g.standard_normal(Lw.shape) * 1e-3
        assert mse((Lw + dl) @ Qw) > mse(Lw @ Qw)


def pin_tau_golden():
    fx = _load("tau_tiny.json")
    P, G = np.array(fx["P"], float), np.array(fx["G"], float)
    for case in fx["cases"]:
        tau = oracle.calibrate_tau(P, G, case["s"])
        assert np.allclose(tau, case["tau"], rtol=0, atol=1e-15), (case, tau)


def pin_tau_monotone():
    """Candidate density never rises with s (tau_i is increasing in s when m+ > m-)."""
    g = np.random.default_rng(20)
    G = g.standard_normal((300, 50)) - 1.0
    P = G + 0.5 * g.standard_normal((300, 50))
    x_p = P[:40]
    prev = None
    for s in (0.0, 0.2, 0.4, 0.5, 0.6, 0.8, 1.0):
        tau = oracle.calibrate_tau(P, G, s)
        dens = oracle.svd_candidates(x_p, tau[None, :]).mean()
        if prev is not None:
            assert dens <= prev + 1e-15
        prev = dens


def pin_effective_density():
    """Hand-computed values of (period rho + rho_verify) / aal."""
    ed = oracle.effective_density
    assert ed(1.0, 16, 16) == 17.0 / 16.0  # a dense "sparse" step: the verification adds 1/16
    assert abs(ed(2.0 / 3.0, 16, 16) - 35.0 / 48.0) <= 1e-15  # CATS at k 0.5 reads 2/3: (32/3 + 1)/16
    assert ed(0.5, 16, 12) == 0.75  # (8 + 1) / 12
    assert ed(0.5, 4, 4, rho_verify=0.0) == 0.5
    for bad in ((0.5, 16, 17), (0.5, 16, 0.0), (0.5, 0, 1)):
        try:
            ed(*bad)
        except ValueError:
            continue
        raise AssertionError(f"accepted {bad}")


def pin_divergence():
    """Hand-worked relative L2 distances, measured against the dense row."""
    dv = oracle.sparse_dense_divergence
    yd = np.array([[3.0, 4.0], [3.0, 4.0], [3.0, 4.0], [0.0, 0.0], [0.0, 0.0]])
    ys = np.array([[3.0, 4.0], [4.5, 6.0], [3.0, 0.0], [0.0, 0.0], [1.0, 0.0]])
    out = dv(ys, yd)
    assert out[0] == 0.0 and out[1] == 0.5 and out[2] == 0.8 and out[3] == 0.0 and np.isinf(out[4])
    assert dv(np.zeros((2, 3)), np.ones((2, 3))).tolist() == [1.0, 1.0]  # nothing active


def pin_period_outputs():
    """A period over two layers: with every neuron active (t = -1) the sparse steps equal
    the verification exactly; with none active (t = inf) they are zero and the
    divergence is 1; each layer's outputs depend on that layer only, and permuting the
    chunk's tokens permutes its rows."""
    g = np.random.default_rng(30)
    d, f, P = 8, 20, 5
    mk = lambda: tuple(g.standard_normal((f, d)) for _ in range(3))  # noqa: E731
    layers = [mk(), mk()]
    X = g.standard_normal((2, P, d))
    ys, yd = oracle.period_outputs(layers, X, [-1.0, -1.0])
    assert ys.shape == (2, P, d) and np.array_equal(ys, yd)
    ys0, yd0 = oracle.period_outputs(layers, X, [np.inf, np.inf])
    assert np.all(ys0 == 0.0) and np.array_equal(yd0, yd)
    assert np.all(oracle.sparse_dense_divergence(ys0, yd0) == 1.0)
    ys1, yd1 = oracle.period_outputs([layers[0], mk()], X, [0.05, 0.05])
    ys2, yd2 = oracle.period_outputs(layers, X, [0.05, 0.05])
    assert np.array_equal(ys1[0], ys2[0]) and np.array_equal(yd1[0], yd2[0])
    perm = g.permutation(P)
    ys3, yd3 = oracle.period_outputs(layers, X[:, perm], [0.05, 0.05])
    assert np.array_equal(ys3, ys2[:, perm]) and np.array_equal(yd3, yd2[:, perm])
    # one token by hand: the dense row is sum_i silu(g_i) u_i Dt[i]
    Wg, Wu, Dt = layers[1]
    x = X[1, 2]
    gg, uu = Wg @ x, Wu @ x
    h = gg / (1.0 + np.exp(-gg)) * uu
    assert np.allclose(yd[1, 2], sum(h[i] * Dt[i] for i in range(f)), rtol=1e-13, atol=1e-13)


def pin_roc_auc_brute_force():
    """Against the definition counted pair by pair (ties one half) on small integer
    scores with many ties."""
    g = np.random.default_rng(31)
    for n in (7, 20, 41):
        sc = g.integers(0, 5, size=n).astype(float)
        lab = g.random(n) < 0.4
        lab[0], lab[1] = True, False
        pos, neg = sc[lab], sc[~lab]
        wins = 0.0
        for a in pos:
            for b in neg:
                wins += 1.0 if a > b else (0.5 if a == b else 0.0)
        assert abs(oracle.roc_auc(sc, lab) - wins / (len(pos) * len(neg))) <= 1e-12


def pin_roc_auc_closed_forms():
    """Separated classes give 1, reversed 0, all tied 1/2; for positives N(mu, 1) against
    negatives N(0, 1) the AUC is Phi(mu / sqrt 2)."""
    lab = np.array([False, False, True, True, True])
    assert oracle.roc_auc([0.1, 0.2, 0.3, 0.4, 0.5], lab) == 1.0
    assert oracle.roc_auc([0.5, 0.4, 0.3, 0.2, 0.1], lab) == 0.0
    assert oracle.roc_auc(np.zeros(5), lab) == 0.5
    g = np.random.default_rng(32)
    for mu in (0.0, 0.5, 1.5):
        neg, pos = g.standard_normal(20000), g.standard_normal(20000) + mu
        auc = oracle.roc_auc(np.concatenate([neg, pos]), np.r_[np.zeros(20000, bool), np.ones(20000, bool)])
        assert abs(auc - stats.norm.cdf(mu / math.sqrt(2.0))) <= 0.01, (mu, auc)


def pin_recall():
    """Hand-worked pooled recall over two tokens."""
    act = np.array([[1, 1, 0, 0, 1], [0, 1, 1, 0, 0]], bool)
    cand = np.array([[1, 0, 1, 0, 1], [0, 1, 0, 1, 0]], bool)
    assert oracle.recall(cand, act) == 3.0 / 5.0
    assert abs(oracle.false_negative_rate(cand, act) - 0.4) <= 1e-15
    assert oracle.recall(np.ones_like(act), act) == 1.0
    # every neuron a candidate: nothing active is dropped (precision would be 5/10)
    assert oracle.false_negative_rate(np.ones_like(act), act) == 0.0


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
