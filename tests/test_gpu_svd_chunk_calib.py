"""GPU parity of svd_predict, ffn_dense_chunk and sparse_ffn_calibrate against the oracle."""

import numpy as np
import pytest
import torch

import oracle
from contextual_activation_sparsity_amd import inputs
from tests.helpers import (TOL_BF16, TOL_F32, check_mask, fp32_output_bound, mask_from_idx, normwise_err,
                           reglu_svd_layer, say, swiglu_layer_dev, to_dev, to_f64)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from contextual_activation_sparsity_amd import binding as B


# ------------------------------------------------------------------------------ SVD
def _svd_case(d, f, r, s, n_tok, n_cal=256, rank_struct=256):
    w = inputs.workload(3)
    say(f"[svd] d={d} f={f} r={r} s={s}")
    raw, Wg, b, Qb, Lb, Q64, L64 = reglu_svd_layer(d, f, r, rank_struct)
    # calibration tokens as the columns of one matrix (the bias broadcast over them)
    xcal = to_f64(inputs.tokens(w, n_cal, inputs.STREAM_TAU, d=d), "bf16").T
    P = oracle.svd_predict(Q64, L64, xcal, b[:, None]).T
    G = oracle.gate_up(Wg, Wg, xcal, b[:, None])[0].T
    tau = oracle.calibrate_tau(P, G, s).astype(np.float32)
    pred = B.SVDPredictor(to_dev(Qb, "bf16"), to_dev(Lb, "bf16"), torch.from_numpy(tau).cuda(),
                          b=torch.from_numpy(raw["b_gate"]).cuda())
    ws = B.workspace(B.svd_predict_workspace_size(pred))
    xs_raw = inputs.tokens(w, n_tok, inputs.STREAM_DECODE, d=d)
    xs = to_f64(xs_raw, "bf16")
    dens = []
    for j in range(n_tok):
        cand = torch.full((f,), -1, dtype=torch.int32, device="cuda")
        n_cand = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        p_out = torch.empty(f, dtype=torch.float32, device="cuda")
        B.svd_predict(pred, to_dev(xs_raw[j], "bf16"), cand, n_cand, ws, p_out=p_out)
        torch.cuda.synchronize()
        p_ref = oracle.svd_predict(Q64, L64, xs[j], b)
        p_gpu = p_out.cpu().numpy()
        scale = np.sqrt((L64 ** 2).sum(1)) * np.linalg.norm(Q64 @ xs[j]) / np.sqrt(r) + 1e-30
        assert np.max(np.abs(p_gpu - p_ref) / (np.abs(p_ref) + scale)) < 1e-4
        nc = int(n_cand.item())
        ci = cand.cpu().numpy()
        assert np.all(np.diff(ci[:nc]) > 0), "candidates ascending"
        cm_ref = oracle.svd_candidates(p_ref, tau)
        check_mask(mask_from_idx(ci, nc, f), cm_ref, p_ref, tau.astype(np.float64), abs_band=1e-3 * scale,
                   what=f"candidates token {j}")
        dens.append(nc / f)
    return raw, pred, ws, (Q64, L64, b, tau), np.array(dens)


@pytest.mark.parametrize("d,f,r", [(512, 1000, 64), (1024, 3000, 128), (2048, 700, 352), (4096, 11008, 256),
                                   (1024, 3000, 520), (4096, 11008, 1024), (8, 8, 8), (16, 70, 8)])
def test_svd_predict(d, f, r):
    _svd_case(d, f, r, 0.5, 3)


def test_svd_sequential_pipeline_end_to_end():
    """svd_predict -> sparse_ffn_decode(cand, ReLU, t=0) against oracle.reglu_sequential."""
    d, f, r = 4096, 11008, 256
    raw, pred, ws_p, (Q64, L64, b, tau), dens = _svd_case(d, f, r, 0.5, 2)
    Wg, Wu, Dt = (to_f64(raw[k], "bf16") for k in ("w_gate", "w_up", "w_down_t"))
    layer = B.FFNLayer(to_dev(raw["w_gate"], "bf16"), to_dev(raw["w_up"], "bf16"), to_dev(raw["w_down_t"], "bf16"),
                       b_gate=torch.from_numpy(raw["b_gate"]).cuda(), act=B.SFN_ACT_RELU)
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, 1))
    w = inputs.workload(3)
    xs_raw = inputs.tokens(w, 2, inputs.STREAM_DECODE, d=d)
    xs = to_f64(xs_raw, "bf16")
    for j in range(2):
        say(f"[svd+decode] token {j}")
        xd = to_dev(xs_raw[j:j + 1], "bf16")
        cand = torch.empty(f, dtype=torch.int32, device="cuda")
        n_cand = torch.empty(1, dtype=torch.int32, device="cuda")
        B.svd_predict(pred, xd, cand, n_cand, ws_p)
        y = torch.empty((1, d), dtype=torch.float32, device="cuda")
        idx = torch.empty((1, f), dtype=torch.int32, device="cuda")
        n_act = torch.empty(1, dtype=torch.int32, device="cuda")
        B.sparse_ffn_decode(layer, xd, None, ws, y=y, cand=cand, n_cand=n_cand, active_idx=idx, n_active=n_act)
        torch.cuda.synchronize()
        cm = mask_from_idx(cand.cpu().numpy(), int(n_cand.item()), f)
        act_gpu = mask_from_idx(idx.cpu().numpy()[0], int(n_act.item()), f)
        active, g, _ = oracle.reglu_sequential(Wg, Wu, Dt, xs[j], cm, b)
        sig = np.sqrt((Wg * Wg).sum(1)) * np.sqrt((xs[j] ** 2).mean())
        check_mask(act_gpu, active, g, 0.0, abs_band=1e-3 * sig)
        _, _, y_own = oracle.reglu_sequential(Wg, Wu, Dt, xs[j], act_gpu, b)
        assert normwise_err(y.cpu().numpy()[0], y_own) <= min(TOL_BF16, fp32_output_bound(Wg, Wu, Dt, xs[j], act_gpu,
                                                                                          "relu", b))
        say(f"    candidates {cm.mean():.3f} active {act_gpu.mean():.3f}")


def test_svd_parallel_pipeline_end_to_end():
    """svd_predict -> sparse_ffn_decode_parallel (ReLU): the oracle's result on the same
    candidates, and the sequential candidate mode's result, within the bf16 tolerance."""
    d, f, r = 4096, 11008, 256
    raw, pred, ws_p, (Q64, L64, b, tau), dens = _svd_case(d, f, r, 0.5, 1)
    Wg, Wu, Dt = (to_f64(raw[k], "bf16") for k in ("w_gate", "w_up", "w_down_t"))
    layer = B.FFNLayer(to_dev(raw["w_gate"], "bf16"), to_dev(raw["w_up"], "bf16"), to_dev(raw["w_down_t"], "bf16"),
                       b_gate=torch.from_numpy(raw["b_gate"]).cuda(), act=B.SFN_ACT_RELU)
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, 1))
    w = inputs.workload(3)
    xs_raw = inputs.tokens(w, 2, inputs.STREAM_DECODE, d=d)
    xs = to_f64(xs_raw, "bf16")
    for j in range(2):
        say(f"[svd+parallel] token {j}")
        xd = to_dev(xs_raw[j:j + 1], "bf16")
        cand = torch.empty(f, dtype=torch.int32, device="cuda")
        n_cand = torch.empty(1, dtype=torch.int32, device="cuda")
        B.svd_predict(pred, xd, cand, n_cand, ws_p)
        y = torch.full((d,), float("nan"), dtype=torch.float32, device="cuda")
        B.sparse_ffn_decode_parallel(layer, xd, cand, n_cand, ws, y)
        ys = torch.empty((1, d), dtype=torch.float32, device="cuda")
        B.sparse_ffn_decode(layer, xd, None, ws, y=ys, cand=cand, n_cand=n_cand)
        torch.cuda.synchronize()
        cm = mask_from_idx(cand.cpu().numpy(), int(n_cand.item()), f)
        _, _, y_ref = oracle.reglu_sequential(Wg, Wu, Dt, xs[j], cm, b)
        assert normwise_err(y.cpu().numpy(), y_ref) <= min(TOL_BF16, fp32_output_bound(Wg, Wu, Dt, xs[j], cm, "relu",
                                                                                       b))
        assert normwise_err(y.cpu().numpy(), ys.cpu().numpy()[0]) <= TOL_BF16


@pytest.mark.parametrize("wi,d,f,act,frac", [(1, 4096, 11008, "silu", 0.3), (1, 1024, 3000, "relu", 0.5),
                                              (1, 8192, 2048, "silu", 0.2), (0, 256, 688, "silu", 0.4),
                                              (1, 2048, 700, "relu", 0.0), (5, 3584, 18944, "silu", 0.05),
                                              (1, 16384, 600, "silu", 0.4)])
def test_parallel_candidate_lists(wi, d, f, act, frac):
    """Unsorted candidate lists of a given fraction of the rows (empty at 0): y is the
    FFN masked to those rows, act(g) u summed against Dt, as the oracle computes it."""
    w = inputs.workload(wi)
    say(f"[parallel] workload={wi} d={d} f={f} act={act} frac={frac}")
    raw, dev, host = swiglu_layer_dev(w, 0, d=d, f=f)
    bias = (np.random.default_rng(5).standard_normal(f) * 0.3).astype(np.float32)
    layer = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"], b_gate=torch.from_numpy(bias).cuda(),
                       act=B.SFN_ACT_SILU if act == "silu" else B.SFN_ACT_RELU)
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, 1))
    xs_raw = inputs.tokens(w, 2, inputs.STREAM_DECODE, d=d)
    xs = to_f64(xs_raw, w.dtype)
    g = np.random.default_rng(6)
    for j in range(2):
        rows = g.permutation(f)[: int(frac * f)].astype(np.int32)
        cand = torch.from_numpy(np.concatenate([rows, np.zeros(f - rows.size, np.int32)])).cuda()
        n_cand = torch.tensor([rows.size], dtype=torch.int32, device="cuda")
        y = torch.full((d,), float("nan"), dtype=torch.float32, device="cuda")
        B.sparse_ffn_decode_parallel(layer, to_dev(xs_raw[j], w.dtype), cand, n_cand, ws, y)
        torch.cuda.synchronize()
        mask = np.zeros(f, bool)
        mask[rows] = True
        y_ref = oracle.masked_ffn(host["w_gate"], host["w_up"], host["w_down_t"], xs[j], mask, act,
                                  bias.astype(np.float64))
        yg = y.cpu().numpy()
        if rows.size == 0:
            assert np.all(yg == 0.0)
        else:
            bnd = fp32_output_bound(host["w_gate"], host["w_up"], host["w_down_t"], xs[j], mask, act,
                                    bias.astype(np.float64))
            assert normwise_err(yg, y_ref) <= min(TOL_BF16 if w.dtype == "bf16" else TOL_F32, bnd)


# ---------------------------------------------------------------------------- chunk
# f > 16384 takes the wide stage 1 (up to 32 rows per workgroup, at most 1024 workgroups):
# f 16400 just past the switch, 20000 with uneven shares, 40000 beyond 1024 full workgroups
@pytest.mark.parametrize("d,f,n", [(4096, 11008, 16), (1024, 3000, 5), (512, 1001, 1), (8192, 2048, 16),
                                   (2048, 4100, 9), (8192, 28672, 16), (4096, 11008, 1), (3584, 18944, 1),
                                   (16384, 300, 16), (256, 16400, 2), (1024, 20000, 5), (512, 40000, 3),
                                   (8, 1, 16), (8, 17, 5)])
def test_dense_chunk_bf16(d, f, n):
    w = inputs.workload(4)
    say(f"[chunk] d={d} f={f} n={n}")
    raw, dev, host = swiglu_layer_dev(w, 0, d=d, f=f)
    layer = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"])
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, 16))
    xs_raw = inputs.tokens(w, n, inputs.STREAM_DECODE, d=d)
    xs = to_f64(xs_raw, "bf16")
    y = torch.full((n, d), float("nan"), dtype=torch.float32, device="cuda")
    B.ffn_dense_chunk(layer, to_dev(xs_raw, "bf16"), y, ws)
    torch.cuda.synchronize()
    Y = y.cpu().numpy()
    Yo = oracle.dense_chunk(host["w_gate"], host["w_up"], host["w_down_t"], xs)
    for j in range(n):
        assert normwise_err(Y[j], Yo[j]) <= TOL_BF16, j
    # a row of the chunk does not depend on the other rows: the last token again, next to
    # the first one, gives the same bits (both on the matrix cores)
    if n >= 2:
        y2 = torch.empty((2, d), dtype=torch.float32, device="cuda")
        B.ffn_dense_chunk(layer, to_dev(xs_raw[[n - 1, 0]], "bf16"), y2, ws)
        torch.cuda.synchronize()
        assert np.array_equal(y2.cpu().numpy()[0].view(np.uint32), Y[n - 1].view(np.uint32))
    # one token alone runs through the decode kernels (threshold 0: every neuron that
    # contributes), with h kept in fp32
    y1 = torch.empty((1, d), dtype=torch.float32, device="cuda")
    B.ffn_dense_chunk(layer, to_dev(xs_raw[n - 1:n], "bf16"), y1, ws)
    torch.cuda.synchronize()
    assert normwise_err(y1.cpu().numpy()[0], Yo[n - 1]) <= TOL_BF16


def test_dense_chunk_f32_and_bias_relu():
    w = inputs.workload(0)
    d, f, n = 256, 688, 7
    say("[chunk] fp32")
    raw, dev, host = swiglu_layer_dev(w, 0, d=d, f=f)
    bias = np.random.default_rng(3).standard_normal(f).astype(np.float32) * 0.1
    for act in ("silu", "relu"):
        layer = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"], b_gate=torch.from_numpy(bias).cuda(),
                           act=B.SFN_ACT_SILU if act == "silu" else B.SFN_ACT_RELU)
        ws = B.workspace(B.sparse_ffn_workspace_size(layer, 16))
        xs_raw = inputs.tokens(w, n, inputs.STREAM_DECODE, d=d)
        y = torch.empty((n, d), dtype=torch.float32, device="cuda")
        B.ffn_dense_chunk(layer, to_dev(xs_raw, "f32"), y, ws)
        torch.cuda.synchronize()
        Yo = oracle.dense_chunk(host["w_gate"], host["w_up"], host["w_down_t"], to_f64(xs_raw, "f32"), act,
                                bias.astype(np.float64))
        for j in range(n):
            assert normwise_err(y.cpu().numpy()[j], Yo[j]) <= TOL_F32


# ---------------------------------------------------------------------- calibration
# Score tiles: 128 tokens per workgroup while ceil(f / 64) < 256, 256 tokens from there on
# (f >= 16321), so the cases span both instances, a partial last neuron tile, a partial
# last token tile (n not a multiple of the tile) and a gate bias.
@pytest.mark.parametrize("wi,d,f,n,k,bias", [(0, 256, 688, 256, 0.5, False), (1, 4096, 11008, 256, 0.5, False),
                                              (1, 4096, 11008, 256, 0.7, False), (1, 1024, 999, 33, 0.3, False),
                                              (1, 512, 700, 20, 0.0, False), (1, 512, 700, 20, 1.0, False),
                                              (1, 1024, 16500, 256, 0.5, False), (1, 512, 16384, 300, 0.5, True),
                                              (2, 4096, 14336, 256, 0.6, False), (4, 8192, 28672, 256, 0.5, False),
                                              (1, 8, 1, 256, 0.5, False), (0, 4, 3, 33, 0.3, True)])
def test_calibrate(wi, d, f, n, k, bias):
    w = inputs.workload(wi)
    say(f"[calibrate] workload={wi} d={d} f={f} n={n} k={k} bias={bias}")
    raw, dev, host = swiglu_layer_dev(w, 0, d=d, f=f)
    b = inputs.rng(inputs.seed(w.index, 0, 9)).standard_normal(f).astype(np.float32) * 0.5 if bias else None
    layer = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"],
                       b_gate=torch.from_numpy(b).cuda() if bias else None)
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, n))
    xcal_raw = inputs.tokens(w, n, inputs.STREAM_CAL, d=d)
    t_out = torch.empty(1, dtype=torch.float32, device="cuda")
    S = torch.empty((n, f), dtype=torch.float32, device="cuda")
    B.sparse_ffn_calibrate(layer, to_dev(xcal_raw, w.dtype), k, t_out, ws, scores_out=S)
    torch.cuda.synchronize()
    t_gpu = float(t_out.item())
    k32 = float(np.float32(k))
    t64, t32, K, S_ref = oracle.calibrate_cats(host["w_gate"], to_f64(xcal_raw, w.dtype), k32,
                                               b.astype(np.float64) if bias else None)
    if K == 0:
        assert t_gpu == -1.0
        return
    if K == S_ref.size:
        assert np.isinf(t_gpu) and t_gpu > 0
        return
    Sg = S.cpu().numpy().astype(np.float64)
    # exact selection on the library's own scores
    assert int((Sg < t_gpu).sum()) < K <= int((Sg <= t_gpu).sum())
    assert t_gpu in set(Sg.ravel().tolist())
    # scores agree with the oracle to fp32 accumulation accuracy ...
    err = np.max(np.abs(Sg - S_ref))
    assert err <= 1e-5 * max(1.0, np.max(S_ref))
    # ... and order statistics are 1-Lipschitz in the max norm
    assert abs(t_gpu - t64) <= err + 1e-7
    # fresh decode tokens (their own seed stream) are cut at the calibrated rate: the
    # library's own masks under its threshold, within 0.02 of k (a statistical check,
    # made only where the 8 tokens hold thousands of neuron decisions)
    n_fresh = 8
    if f * n_fresh < 4000:
        return
    xs_raw = inputs.tokens(w, n_fresh, inputs.STREAM_DECODE, d=d)
    na = torch.empty(1, dtype=torch.int32, device="cuda")
    ia = torch.empty((1, f), dtype=torch.int32, device="cuda")
    dens = []
    for j in range(n_fresh):
        B.sparse_ffn_decode(layer, to_dev(xs_raw[j:j + 1], w.dtype), t_out, ws, active_idx=ia, n_active=na)
        torch.cuda.synchronize()
        dens.append(int(na.item()) / f)
    say(f"    t {t_gpu:.5f} (oracle {t64:.5f}); fresh-token sparsity {1.0 - np.mean(dens):.4f}")
    assert abs((1.0 - np.mean(dens)) - k) <= 0.02, dens
