"""Every library call captured in one HIP graph (as the benchmark runs them) and replayed
several times, with the program's own eager work and synchronizations in between: each
replay must reproduce the eager outputs bit for bit. All calls share one workspace, as
consecutive calls on one stream may."""

import numpy as np
import pytest
import torch

import oracle
from contextual_activation_sparsity_amd import inputs
from tests.helpers import say, swiglu_layer_dev, to_dev, to_f64

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from contextual_activation_sparsity_amd import binding as B


def test_graph_replays_match_eager():
    w1, w3 = inputs.workload(1), inputs.workload(3)
    d, f, r = 1024, 3000, 128
    say(f"[graph] d={d} f={f} r={r}")
    raw, dev, host = swiglu_layer_dev(w1, 0, d=d, f=f)
    swi = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"])
    rg = inputs.reglu_layer(w3, 0, d=d, f=f, rank_struct=256)
    bdev = torch.from_numpy(rg["b_gate"]).cuda()
    reg = B.FFNLayer(to_dev(rg["w_gate"], "bf16"), to_dev(rg["w_up"], "bf16"), to_dev(rg["w_down_t"], "bf16"),
                     b_gate=bdev, act=B.SFN_ACT_RELU)
    Wg = to_f64(rg["w_gate"], "bf16")
    Q, L = oracle.svd_factors(Wg, r)
    tau = np.zeros(f, np.float32)
    pred = B.SVDPredictor(to_dev(inputs.f32_to_bf16_bits(Q), "bf16"), to_dev(inputs.f32_to_bf16_bits(L), "bf16"),
                          torch.from_numpy(tau).cuda(), b=bdev)
    ws = B.workspace(max(B.sparse_ffn_workspace_size(swi, 256), B.sparse_ffn_workspace_size(reg, 16),
                         B.svd_predict_workspace_size(pred), B.sparse_ffn_svd_workspace_size(reg, pred)))
    xcal = to_dev(inputs.tokens(w1, 256, inputs.STREAM_CAL, d=d), "bf16")
    X = to_dev(inputs.tokens(w1, 16, inputs.STREAM_DECODE, d=d), "bf16")
    cuda = dict(device="cuda")
    out = {
        "t": torch.empty(1, dtype=torch.float32, **cuda),
        "y1": torch.empty((1, d), dtype=torch.float32, **cuda),
        "i1": torch.empty((1, f), dtype=torch.int32, **cuda), "n1": torch.empty(1, dtype=torch.int32, **cuda),
        "y4": torch.empty((4, d), dtype=torch.float32, **cuda),
        "Y16": torch.empty((16, d), dtype=torch.float32, **cuda),
        "cand": torch.empty(f, dtype=torch.int32, **cuda), "nc": torch.empty(1, dtype=torch.int32, **cuda),
        "p": torch.empty(f, dtype=torch.float32, **cuda),
        "yc": torch.empty((1, d), dtype=torch.float32, **cuda),
        "yp": torch.empty(d, dtype=torch.float32, **cuda),
        "ys": torch.empty(d, dtype=torch.float32, **cuda),
        "is": torch.empty(f, dtype=torch.int32, **cuda), "ns": torch.empty(1, dtype=torch.int32, **cuda),
        "yq": torch.empty(d, dtype=torch.float32, **cuda),
    }

    def calls():
        B.sparse_ffn_calibrate(swi, xcal, 0.5, out["t"], ws)
        B.sparse_ffn_decode(swi, X[:1], out["t"], ws, y=out["y1"], active_idx=out["i1"], n_active=out["n1"])
        B.sparse_ffn_decode(swi, X[1:5], out["t"], ws, y=out["y4"])
        B.ffn_dense_chunk(swi, X, out["Y16"], ws)
        B.svd_predict(pred, X[5:6], out["cand"], out["nc"], ws, p_out=out["p"])
        B.sparse_ffn_decode(reg, X[5:6], None, ws, y=out["yc"], cand=out["cand"], n_cand=out["nc"])
        B.sparse_ffn_decode_parallel(reg, X[5:6], out["cand"], out["nc"], ws, out["yp"])
        B.sparse_ffn_decode_svd(reg, pred, X[6:7], ws, y=out["ys"], idx=out["is"], n_idx=out["ns"],
                                pipeline=B.SFN_PIPE_SEQUENTIAL)
        B.sparse_ffn_decode_svd(reg, pred, X[7:8], ws, y=out["yq"], pipeline=B.SFN_PIPE_PARALLEL)

    def poison():
        for v in out.values():
            v.fill_(-7 if v.dtype == torch.int32 else float("nan"))

    poison()
    calls()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in out.items()}
    assert 0 < int(ref["n1"].item()) < f and 0 < int(ref["nc"].item()) < f and 0 < int(ref["ns"].item()) < f
    g = torch.cuda.CUDAGraph()
    poison()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        poison()
        # the program's own eager work between replays
        junk = torch.randn((512, 512), **cuda) @ torch.randn((512, 512), **cuda)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        del junk
        for k, v in out.items():
            assert torch.equal(v, ref[k]), f"replay {rep}: {k} differs from the eager result"
        assert not bool(ws[:B.SFN_WORKSPACE_HEADER_BYTES].any().item())


def test_graph_replays_balanced_one_token():
    """One-token calls with rows wider than 8 KB (the tiles balance their up/down rows
    through count words in the workspace header, zeroed again by each call's last kernel)
    captured back to back in one graph, several layers on one workspace: every replay
    reproduces the eager outputs bit for bit and leaves the header zero."""
    w = inputs.workload(4)
    d, f, n_layers = 8192, 3000, 3
    say(f"[graph balanced] d={d} f={f} layers={n_layers}")
    layers = []
    for l in range(n_layers):
        raw, dev, host = swiglu_layer_dev(w, l, d=d, f=f)
        layers.append(B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"]))
    ws = B.workspace(B.sparse_ffn_workspace_size(layers[0], 1))
    X = to_dev(inputs.tokens(w, n_layers, inputs.STREAM_DECODE, d=d), "bf16")
    t = torch.full((1,), 0.02, dtype=torch.float32, device="cuda")
    Y = torch.empty((n_layers, d), dtype=torch.float32, device="cuda")
    I = torch.empty((n_layers, f), dtype=torch.int32, device="cuda")
    N = torch.empty((n_layers,), dtype=torch.int32, device="cuda")

    def calls():
        for l in range(n_layers):
            B.sparse_ffn_decode(layers[l], X[l:l + 1], t, ws, y=Y[l:l + 1], active_idx=I[l:l + 1],
                                n_active=N[l:l + 1])

    def poison():
        Y.fill_(float("nan"))
        I.fill_(-7)
        N.fill_(-7)

    poison()
    calls()
    torch.cuda.synchronize()
    ref = (Y.clone(), I.clone(), N.clone())
    assert bool((ref[2] > 0).all()) and bool((ref[2] < f).all())
    g = torch.cuda.CUDAGraph()
    poison()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        poison()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(Y, ref[0]) and torch.equal(I, ref[1]) and torch.equal(N, ref[2]), rep
        assert not bool(ws[:B.SFN_WORKSPACE_HEADER_BYTES].any().item())
