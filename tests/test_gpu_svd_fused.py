"""GPU parity of sparse_ffn_decode_svd: the SVD predictor and the FFN in one call, each
tile processing the candidates among its own rows ("SVD Contextual Sparsity Predictors
for Fast LLM Inference", Figures 1 and 3, Table 2), for both pipelines.

Against the oracle (oracle.svd_predict, svd_candidates, reglu_sequential): candidates
{p > tau} with p = L (Q x) + b in float64, and for the sequential pipeline the actives
{candidates with g > 0}. Sets must agree except where p
is within rounding of tau or g within rounding of 0 (at most 0.1% of the rows). y is
compared with the oracle's FFN on the library's own set. The fused call is also compared
with the unfused one (svd_predict, then the candidate-mode or one-pass decode).
"""

import numpy as np
import pytest
import torch

import oracle
from contextual_activation_sparsity_amd import inputs
from tests.helpers import TOL_BF16, fp32_output_bound, mask_from_idx, normwise_err, reglu_svd_layer, say, to_dev, to_f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from contextual_activation_sparsity_amd import binding as B

BAND = 1e-3


def _setup(d, f, r, s=0.5, act="relu", tau_override=None):
    w = inputs.workload(3)
    raw, Wg, b, Qb, Lb, Q64, L64 = reglu_svd_layer(d, f, r, min(256, d, f))
    Wu, Dt = (to_f64(raw[k], "bf16") for k in ("w_up", "w_down_t"))
    if tau_override is None:
        # calibration tokens as the columns of one matrix: the oracle's predictor and gate
        # evaluate all of them in one product (the bias broadcast over the columns)
        xcal = to_f64(inputs.tokens(w, 512, inputs.STREAM_TAU, d=d), "bf16").T
        P = oracle.svd_predict(Q64, L64, xcal, b[:, None]).T
        G = oracle.gate_up(Wg, Wu, xcal, b[:, None])[0].T
        tau = oracle.calibrate_tau(P, G, s).astype(np.float32)
    else:
        tau = np.full(f, tau_override, dtype=np.float32)
    bdev = torch.from_numpy(raw["b_gate"]).cuda()
    layer = B.FFNLayer(to_dev(raw["w_gate"], "bf16"), to_dev(raw["w_up"], "bf16"), to_dev(raw["w_down_t"], "bf16"),
                       b_gate=bdev, act=B.SFN_ACT_RELU if act == "relu" else B.SFN_ACT_SILU)
    pred = B.SVDPredictor(to_dev(Qb, "bf16"), to_dev(Lb, "bf16"), torch.from_numpy(tau).cuda(), b=bdev)
    return w, (Wg, Wu, Dt, b, Q64, L64, tau.astype(np.float64)), layer, pred


def _p_band(Q64, L64, x, tau, r):
    """Rounding scale of a float32 prediction: |L_i| |Q x| / sqrt(r) (the size of one
    row's dot product with the projected token) plus |tau_i|, times the band."""
    return BAND * (np.sqrt((L64 ** 2).sum(1)) * np.linalg.norm(Q64 @ x) / np.sqrt(r) + np.abs(tau))


def _g_band(Wg, x):
    """Rounding scale of a float32 gate around the ReLU threshold 0: |w_i| rms(x)."""
    return BAND * np.sqrt((Wg * Wg).sum(1)) * np.sqrt((x * x).mean())


def _check_set(gpu, ref, near, what):
    bad = gpu != ref
    outside = bad & ~near
    assert not outside.any(), f"{what}: {int(outside.sum())} mismatches outside the band"
    assert bad.sum() <= max(2, 1e-3 * bad.size), f"{what}: {int(bad.sum())} band mismatches"
    return int(bad.sum())


def _run(layer, pred, xd, pipeline, want_y=True):
    f, d = layer.f, layer.d
    ws = B.workspace(B.sparse_ffn_svd_workspace_size(layer, pred))
    y = torch.full((d,), float("nan"), dtype=torch.float32, device="cuda") if want_y else None
    idx = torch.full((f,), -1, dtype=torch.int32, device="cuda")
    n = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    B.sparse_ffn_decode_svd(layer, pred, xd, ws, y=y, idx=idx, n_idx=n, pipeline=pipeline)
    torch.cuda.synchronize()
    assert not bool(ws[:B.SFN_WORKSPACE_HEADER_BYTES].any().item()), "reserved workspace header changed"
    nn = int(n.item())
    ii = idx.cpu().numpy()
    assert 0 <= nn <= f and np.all(np.diff(ii[:nn]) > 0), "ascending rows"
    return (y.cpu().numpy() if want_y else None), mask_from_idx(ii, nn, f)


@pytest.mark.parametrize("d,f,r", [(4096, 11008, 256), (1024, 3000, 128), (512, 1000, 64), (256, 70000, 64),
                                   (8192, 2048, 512), (512, 1000, 8), (4096, 11008, 1024), (8, 8, 8),
                                   (16, 70, 8)])
def test_sequential_matches_oracle(d, f, r):
    say(f"[svd fused seq] d={d} f={f} r={r}")
    w, (Wg, Wu, Dt, b, Q64, L64, tau), layer, pred = _setup(d, f, r)
    xs_raw = inputs.tokens(w, 2, inputs.STREAM_DECODE, d=d)
    xs = to_f64(xs_raw, "bf16")
    for j in range(2):
        x = xs[j]
        y, act_gpu = _run(layer, pred, to_dev(xs_raw[j:j + 1], "bf16"), B.SFN_PIPE_SEQUENTIAL)
        p = oracle.svd_predict(Q64, L64, x, b)
        ref, g, _ = oracle.reglu_sequential(Wg, Wu, Dt, x, oracle.svd_candidates(p, tau), b)
        near = (np.abs(p - tau) <= _p_band(Q64, L64, x, tau, r)) | (np.abs(g) <= _g_band(Wg, x))
        mism = _check_set(act_gpu, ref, near, f"actives token {j}")
        # y on the library's own active set (ReLU zeroes the rest, so it is the same set)
        _, _, y_own = oracle.reglu_sequential(Wg, Wu, Dt, x, act_gpu, b)
        assert normwise_err(y, y_own) <= min(TOL_BF16, fp32_output_bound(Wg, Wu, Dt, x, act_gpu, "relu", b))
        say(f"    actives {act_gpu.mean():.4f} (band mismatches {mism})")


@pytest.mark.parametrize("d,f,r,act", [(4096, 11008, 1024, "relu"), (4096, 11008, 256, "silu"),
                                       (1024, 3000, 128, "relu"), (256, 70000, 64, "silu"), (512, 1000, 8, "relu"),
                                       (8, 8, 8, "relu"), (16, 70, 8, "silu")])
def test_parallel_matches_oracle(d, f, r, act):
    say(f"[svd fused par] d={d} f={f} r={r} act={act}")
    w, (Wg, Wu, Dt, b, Q64, L64, tau), layer, pred = _setup(d, f, r, act=act)
    xs_raw = inputs.tokens(w, 2, inputs.STREAM_DECODE, d=d)
    xs = to_f64(xs_raw, "bf16")
    for j in range(2):
        x = xs[j]
        y, cand_gpu = _run(layer, pred, to_dev(xs_raw[j:j + 1], "bf16"), B.SFN_PIPE_PARALLEL)
        p = oracle.svd_predict(Q64, L64, x, b)
        mism = _check_set(cand_gpu, oracle.svd_candidates(p, tau), np.abs(p - tau) <= _p_band(Q64, L64, x, tau, r),
                          f"candidates token {j}")
        y_own = oracle.masked_ffn(Wg, Wu, Dt, x, cand_gpu, act, b)
        assert normwise_err(y, y_own) <= min(TOL_BF16, fp32_output_bound(Wg, Wu, Dt, x, cand_gpu, act, b))
        say(f"    candidates {cand_gpu.mean():.4f} (band mismatches {mism})")


def test_fused_equals_unfused():
    """The same layer through svd_predict + sparse_ffn_decode(cand) / _parallel: the row
    sets agree up to predictions within rounding of tau, and y within tolerance when the
    sets agree."""
    d, f, r = 4096, 11008, 256
    w, (Wg, Wu, Dt, b, Q64, L64, tau), layer, pred = _setup(d, f, r)
    xs_raw = inputs.tokens(w, 3, inputs.STREAM_DECODE, d=d)
    ws_p = B.workspace(B.svd_predict_workspace_size(pred))
    ws_d = B.workspace(B.sparse_ffn_workspace_size(layer, 1))
    for j in range(3):
        xd = to_dev(xs_raw[j:j + 1], "bf16")
        cand = torch.empty(f, dtype=torch.int32, device="cuda")
        nc = torch.empty(1, dtype=torch.int32, device="cuda")
        B.svd_predict(pred, xd, cand, nc, ws_p)
        ys = torch.empty((1, d), dtype=torch.float32, device="cuda")
        ia = torch.empty((1, f), dtype=torch.int32, device="cuda")
        na = torch.empty(1, dtype=torch.int32, device="cuda")
        B.sparse_ffn_decode(layer, xd, None, ws_d, y=ys, cand=cand, n_cand=nc, active_idx=ia, n_active=na)
        yp = torch.empty(d, dtype=torch.float32, device="cuda")
        B.sparse_ffn_decode_parallel(layer, xd, cand, nc, ws_d, yp)
        torch.cuda.synchronize()
        y_seq, act_f = _run(layer, pred, xd, B.SFN_PIPE_SEQUENTIAL)
        y_par, cand_f = _run(layer, pred, xd, B.SFN_PIPE_PARALLEL)
        cand_u = mask_from_idx(cand.cpu().numpy(), int(nc.item()), f)
        act_u = mask_from_idx(ia.cpu().numpy()[0], int(na.item()), f)
        assert (cand_u != cand_f).sum() <= 2 and (act_u != act_f).sum() <= 2
        if np.array_equal(act_u, act_f):
            assert normwise_err(y_seq, ys.cpu().numpy()[0]) <= 1e-5
        if np.array_equal(cand_u, cand_f):
            assert normwise_err(y_par, yp.cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("pipeline", [0, 1])
def test_no_candidates_and_all_candidates(pipeline):
    """tau = +inf: no candidate, y = 0 and no rows; tau = -inf: every row a candidate, so
    the sequential pipeline is the dense ReGLU FFN and the parallel one the dense FFN."""
    d, f, r = 1024, 3000, 64
    for tv in (np.inf, -np.inf):
        w, (Wg, Wu, Dt, b, Q64, L64, tau), layer, pred = _setup(d, f, r, tau_override=tv)
        xs_raw = inputs.tokens(w, 1, inputs.STREAM_DECODE, d=d)
        y, rows = _run(layer, pred, to_dev(xs_raw, "bf16"), pipeline)
        x = to_f64(xs_raw, "bf16")[0]
        if tv == np.inf:
            assert not rows.any() and np.all(y == 0.0)
        else:
            active, g, _ = oracle.reglu_sequential(Wg, Wu, Dt, x, np.ones(f, bool), b)
            expect = active if pipeline == 0 else np.ones(f, bool)
            near = np.abs(g) <= _g_band(Wg, x)
            _check_set(rows, expect, near if pipeline == 0 else np.zeros(f, bool), "rows")
            assert normwise_err(y, oracle.dense_ffn(Wg, Wu, Dt, x, "relu", b)) <= TOL_BF16


def test_sequential_mask_only():
    """y = NULL: the active rows alone (gate pass and index assembly, no up/down)."""
    d, f, r = 1024, 3000, 128
    w, (Wg, Wu, Dt, b, Q64, L64, tau), layer, pred = _setup(d, f, r)
    xs_raw = inputs.tokens(w, 1, inputs.STREAM_DECODE, d=d)
    xd = to_dev(xs_raw, "bf16")
    _, rows_y = _run(layer, pred, xd, B.SFN_PIPE_SEQUENTIAL)
    _, rows_m = _run(layer, pred, xd, B.SFN_PIPE_SEQUENTIAL, want_y=False)
    assert np.array_equal(rows_y, rows_m)
