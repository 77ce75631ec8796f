"""sparse_ffn_decode_noalloc (the decode step on the library's fixed device scratch, for
callers that cannot allocate) against sparse_ffn_decode on a workspace: the same
kernels and launch shapes, so y, the active index lists and their counts must match bit
for bit. Three calls in a row on the shared scratch: a Llama-2-7B-shaped layer (one
token), then a smaller layer with a batch of three tokens, then the first layer again."""

import numpy as np
import pytest
import torch

from contextual_activation_sparsity_amd import inputs
from tests.helpers import say, swiglu_layer_dev, to_dev

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from contextual_activation_sparsity_amd import binding as B


def _both(layer, x_dev, t_val, nb):
    d, f = layer.d, layer.f
    t = torch.tensor([t_val], dtype=torch.float32, device="cuda")
    out = []
    for noalloc in (False, True):
        y = torch.full((nb, d), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((nb, f), -1, dtype=torch.int32, device="cuda")
        n = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
        if noalloc:
            B.sparse_ffn_decode_noalloc(layer, x_dev, t, y=y, active_idx=idx, n_active=n)
        else:
            ws = B.workspace(B.sparse_ffn_workspace_size(layer, nb))
            B.sparse_ffn_decode(layer, x_dev, t, ws, y=y, active_idx=idx, n_active=n)
        torch.cuda.synchronize()
        out.append((y.cpu().numpy(), idx.cpu().numpy(), n.cpu().numpy()))
    return out


def _check(a, b, what):
    (ya, ia, na), (yb, ib, nb_) = a, b
    assert np.array_equal(na, nb_), (what, na, nb_)
    for j in range(na.shape[0]):
        assert 0 < na[j] < ia.shape[1], (what, na)
        assert np.array_equal(ia[j, :na[j]], ib[j, :nb_[j]]), what
    assert not np.isnan(ya).any()
    assert np.array_equal(ya.view(np.uint32), yb.view(np.uint32)), (what, np.max(np.abs(ya - yb)))


def test_noalloc_matches_workspace_decode():
    w = inputs.workload(1)
    cases = [(4096, 11008, 1), (1024, 2000, 3), (4096, 11008, 1)]
    layers = {}
    for i, (d, f, nb) in enumerate(cases):
        say(f"[noalloc] call {i}: d={d} f={f} batch={nb}")
        if (d, f) not in layers:
            raw, dev, _ = swiglu_layer_dev(w, 0, d=d, f=f)
            layers[(d, f)] = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"])
        layer = layers[(d, f)]
        xs = to_dev(inputs.tokens(w, nb, inputs.STREAM_DECODE, d=d), "bf16")
        a, b = _both(layer, xs, 0.265, nb)
        _check(a, b, f"call {i}")
        say(f"    active {a[2].tolist()} of {f}: identical")


def test_noalloc_in_a_graph():
    """Graph capture, the use the allocation-free call exists for: one call at 8 KB rows
    and one at d 8192 (whose tiles balance through the scratch array's header) captured in
    one graph, replayed three times with workspace calls in between; every replay gives
    the eager results bit for bit. An eager call comes first, so the array's address is
    already resolved when capture starts."""
    w = inputs.workload(1)
    cases = [(4096, 11008), (8192, 6000)]
    layers, xs, ys, want = [], [], [], []
    t = torch.tensor([0.265], dtype=torch.float32, device="cuda")
    for d, f in cases:
        raw, dev, _ = swiglu_layer_dev(w, 2, d=d, f=f)
        layer = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"])
        x = to_dev(inputs.tokens(w, 1, inputs.STREAM_DECODE, d=d), "bf16")
        y = torch.full((1, d), float("nan"), dtype=torch.float32, device="cuda")
        B.sparse_ffn_decode_noalloc(layer, x, t, y=y)
        torch.cuda.synchronize()
        layers.append(layer)
        xs.append(x)
        ys.append(y)
        want.append(y.clone())
    other = B.FFNLayer(*swiglu_layer_dev(w, 3, d=1024, f=2000)[1].values())
    ws = B.workspace(B.sparse_ffn_workspace_size(other, 4))
    x4 = to_dev(inputs.tokens(w, 4, inputs.STREAM_CAL, d=1024), "bf16")
    y4 = torch.empty((4, 1024), dtype=torch.float32, device="cuda")
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    for y in ys:
        y.fill_(float("nan"))
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cap):
        for layer, x, y in zip(layers, xs, ys):
            B.sparse_ffn_decode_noalloc(layer, x, t, y=y, stream=cap)
    for rep in range(3):
        say(f"[noalloc graph] replay {rep}")
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for (d, f), y, yw in zip(cases, ys, want):
            assert torch.equal(y.view(torch.int32), yw.view(torch.int32)), (rep, d, f)
        B.sparse_ffn_decode(other, x4, t, ws, y=y4)  # eager work between the replays
        torch.cuda.synchronize()
