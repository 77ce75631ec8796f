"""GPU parity of sparse_ffn_decode against the CPU oracle (dense FFN, then mask).

Each case draws seeded synthetic inputs, runs the library through the C ABI and checks:
  * active sets: equal to the oracle's except for scores within 1e-3 relative of the
    threshold, at most 0.1% of the neurons;
  * outputs on the oracle's own mask (passed in as the mask override): normwise error
    <= 2e-3 (fp32 weights) / 1e-2 (bf16 weights), fp32 accumulation;
  * outputs on the library's own mask against the oracle on that same mask;
  * both outputs also within the fp32 accumulation bound of tests.helpers, far below the
    contract, so that a dropped or repeated row fails even where 1e-2 would pass it.
"""

import numpy as np
import pytest
import torch

import oracle
from contextual_activation_sparsity_amd import inputs
from tests.helpers import (TOL_BF16, TOL_F32, check_mask, fp32_output_bound, mask_from_idx, normwise_err, say,
                           swiglu_layer_dev, to_dev, to_f64)

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from contextual_activation_sparsity_amd import binding as B


def _tol(dtype):
    return TOL_BF16 if dtype == "bf16" else TOL_F32


def _header_clear(ws):
    """The reserved header of a workspace is zero whenever no call is in flight."""
    return not bool(ws[:B.SFN_WORKSPACE_HEADER_BYTES].any().item())


def run_decode(layer, x_dev, t_val, ws, mask=None, want_y=True, cand=None, n_cand=None):
    Bn = x_dev.shape[0]
    t = torch.tensor([t_val], dtype=torch.float32, device="cuda") if t_val is not None else None
    y = torch.full((Bn, layer.d), float("nan"), dtype=torch.float32, device="cuda") if want_y else None
    idx = torch.full((Bn, layer.f), -1, dtype=torch.int32, device="cuda")
    n_act = torch.full((Bn,), -1, dtype=torch.int32, device="cuda")
    m = torch.from_numpy(np.ascontiguousarray(mask, dtype=np.uint8)).cuda() if mask is not None else None
    B.sparse_ffn_decode(layer, x_dev, t, ws, y=y, mask_in=m, active_idx=idx, n_active=n_act, cand=cand,
                        n_cand=n_cand)
    torch.cuda.synchronize()
    assert _header_clear(ws)
    return (y.cpu().numpy() if want_y else None), idx.cpu().numpy(), n_act.cpu().numpy()


def _case(w, d, f, k, n_tok, seed_layer=0, batch=1, act="silu"):
    """Calibrate t with the oracle on the workload's calibration tokens, run n_tok
    decode tokens in batches, compare with the oracle."""
    say(f"[decode] workload={w.name} d={d} f={f} k={k} tokens={n_tok} batch={batch}")
    raw, dev, host = swiglu_layer_dev(w, seed_layer, d=d, f=f)
    Wg, Wu, Dt = host["w_gate"], host["w_up"], host["w_down_t"]
    xcal = to_f64(inputs.tokens(w, w.n_cal, inputs.STREAM_CAL, d=d), w.dtype)
    _, t32, K, _ = oracle.calibrate_cats(Wg, xcal, k)
    t = float(t32)
    xs_raw = inputs.tokens(w, n_tok, inputs.STREAM_DECODE, d=d)
    xs = to_f64(xs_raw, w.dtype)
    layer = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"],
                       act=B.SFN_ACT_SILU if act == "silu" else B.SFN_ACT_RELU)
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, batch))
    tol = _tol(w.dtype)
    worst = 0.0
    mism = 0
    for j0 in range(0, n_tok, batch):
        xb = xs[j0:j0 + batch]
        xd = to_dev(xs_raw[j0:j0 + batch], w.dtype)
        om, oa, _ = oracle.cats_decode(Wg, Wu, Dt, xb, t, act=act)
        y, idx, n_act = run_decode(layer, xd, t, ws)
        for b in range(xb.shape[0]):
            gm = mask_from_idx(idx[b], n_act[b], f)
            assert np.all(np.diff(idx[b][:n_act[b]]) > 0), "active indices ascending"
            mism += check_mask(gm, om[b], np.abs(oa[b]), t, what=f"token {j0 + b}")
            # own mask: compare with the oracle on the library's mask
            y_own = oracle.masked_ffn(Wg, Wu, Dt, xb[b], gm, act)
            e1 = normwise_err(y[b], y_own)
            bnd = fp32_output_bound(Wg, Wu, Dt, xb[b], gm, act)
            assert e1 <= min(tol, bnd), (j0 + b, e1, bnd)
            worst = max(worst, e1)
        # oracle's mask through the override
        y2, idx2, n2 = run_decode(layer, xd, t, ws, mask=om.astype(np.uint8))
        for b in range(xb.shape[0]):
            yo = oracle.masked_ffn(Wg, Wu, Dt, xb[b], om[b], act)
            e2 = normwise_err(y2[b], yo)
            assert e2 <= min(tol, fp32_output_bound(Wg, Wu, Dt, xb[b], om[b], act)), (j0 + b, e2)
            assert n2[b] == om[b].sum()
            assert np.array_equal(np.sort(idx2[b][:n2[b]]), np.flatnonzero(om[b]))
    say(f"    worst normwise err {worst:.3e}, band mismatches {mism}")
    return layer, ws, dev, host, t


def test_tiny_fp32_all_tokens():
    w = inputs.workload(0)
    _case(w, w.d, w.f, 0.5, w.decode_tokens)


@pytest.mark.parametrize("d,f", [(512, 1000), (1024, 777), (128, 300), (8192, 2000), (2048, 4099)])
def test_ragged_shapes_bf16(d, f):
    w = inputs.workload(1)
    _case(w, d, f, 0.5, 4)


@pytest.mark.parametrize("d,f", [(96, 500), (1024, 1030), (2048, 3000), (4096, 2500), (8192, 1500)])
def test_ragged_shapes_f32(d, f):
    """fp32 rows of up to 32 KB; from 16 KB (d 4096) on, one token takes the balanced
    per-tile up/down."""
    w = inputs.workload(0)
    _case(w, d, f, 0.6, 4)


@pytest.mark.parametrize("dtype_w,d,f,batch", [(1, 256, 70000, 1), (1, 256, 70000, 4), (0, 96, 700, 3),
                                               (0, 1024, 1030, 4)])
def test_wide_layers_and_f32_batches(dtype_w, d, f, batch):
    """More than 65536 neurons (tiles of 256 rows; batches then fall back to the vector
    gate, past the matrix-core gate's 1024 tiles), and fp32 batches (vector gate)."""
    w = inputs.workload(dtype_w)
    _case(w, d, f, 0.5, 2 * batch, batch=batch)


@pytest.mark.parametrize("d,f,batch", [(40, 504, 1), (512, 512, 1), (512, 520, 1), (128, 2040, 1), (64, 65800, 1),
                                       (40, 520, 3)])
def test_partial_row_counts_around_reduce_rounds(d, f, batch):
    """Partial-row counts on either side of the reduce kernel's rounds of 64 and 256 rows
    (63, 64, 65, 255 and 258 workgroups, one partial row each), and rows whose 32-column
    chunks end part-way (d 40): against the oracle within the fp32 bound, which a dropped
    or doubled partial row exceeds, and bitwise the same over repeated calls."""
    w = inputs.workload(1)
    layer, ws, _, _, t = _case(w, d, f, 0.5, 2 * batch, batch=batch)
    xd = to_dev(inputs.tokens(w, batch, inputs.STREAM_DECODE, d=d), w.dtype)
    y_a, idx_a, n_a = run_decode(layer, xd, t, ws)
    for _ in range(2):
        y_b, idx_b, n_b = run_decode(layer, xd, t, ws)
        assert np.array_equal(y_a.view(np.uint32), y_b.view(np.uint32))
        assert np.array_equal(idx_a, idx_b) and np.array_equal(n_a, n_b)


@pytest.mark.parametrize("dtype_w,d,f,batch", [(1, 8, 1, 1), (1, 8, 17, 4), (1, 16, 3, 2), (0, 4, 5, 1),
                                               (0, 4, 2, 3)])
def test_degenerate_shapes(dtype_w, d, f, batch):
    """The smallest layers: rows of one 16-byte chunk (d 8 in bf16, d 4 in fp32), a
    single neuron, tiles with one or no rows, batches on the matrix-core gate whose tiles
    are mostly empty."""
    w = inputs.workload(dtype_w)
    _case(w, d, f, 0.5, 2 * batch, batch=batch)


@pytest.mark.parametrize("k", [0.5, 0.7])
def test_llama2_7b_layer(k):
    w = inputs.workload(1)
    _case(w, w.d, w.f, k, 4)


def test_llama3_70b_layer():
    """Full Llama-3-70B FFN shape (d 8192: two 16-byte chunks per thread and row)."""
    w = inputs.workload(4)
    _case(w, w.d, w.f, 0.5, 2)


@pytest.mark.parametrize("d,f,k", [(8192, 6000, 0.5), (5120, 7000, 0.8)])
def test_balanced_tiles_determinism_and_shared_workspace(d, f, k):
    """One token with rows wider than 8 KB: the tiles balance their up/down rows through
    count words in the workspace header. Against the oracle (in _case); then y and the
    index lists bitwise equal over repeated calls, also when calls of other kinds (a batch
    of four, calibration, the dense chunk) use the same workspace in between, and the
    header zero after every call."""
    w = inputs.workload(4)
    layer, _, dev, host, t = _case(w, d, f, k, 2)
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, 16))
    xs_raw = inputs.tokens(w, 5, inputs.STREAM_DECODE, d=d)
    x1, x4 = to_dev(xs_raw[:1], w.dtype), to_dev(xs_raw[1:5], w.dtype)
    xc = to_dev(inputs.tokens(w, 16, inputs.STREAM_CAL, d=d), w.dtype)
    t_out = torch.zeros(1, dtype=torch.float32, device="cuda")
    y16 = torch.empty((16, d), dtype=torch.float32, device="cuda")
    y0, i0, n0 = run_decode(layer, x1, t, ws)
    for rep in range(3):
        say(f"    repeat {rep}")
        run_decode(layer, x4, t, ws)
        B.sparse_ffn_calibrate(layer, xc, k, t_out, ws)
        B.ffn_dense_chunk(layer, xc, y16, ws)
        torch.cuda.synchronize()
        assert _header_clear(ws)
        y1, i1, n1 = run_decode(layer, x1, t, ws)
        assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
        assert n0[0] == n1[0] and np.array_equal(i0[0][:n0[0]], i1[0][:n1[0]])


def test_balanced_tiles_uneven_counts():
    """The balancer's hand-offs under very uneven tiles (rows wider than 8 KB, mask
    override): every active row in the first tiles, one active row, every row active,
    and a comb that leaves alternate tiles empty. y against the oracle on the same mask,
    bitwise equal on a second call, header zero after each call."""
    w = inputs.workload(4)
    d, f = 8192, 4000
    raw, dev, host = swiglu_layer_dev(w, 0, d=d, f=f)
    Wg, Wu, Dt = host["w_gate"], host["w_up"], host["w_down_t"]
    layer = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"])
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, 1))
    x_raw = inputs.tokens(w, 1, inputs.STREAM_DECODE, d=d)
    x = to_f64(x_raw, w.dtype)[0]
    xd = to_dev(x_raw, w.dtype)
    rows_per_tile = f / 256
    masks = {"first tiles": np.arange(f) < 300, "one row": np.arange(f) == 2345, "all": np.ones(f, bool),
             "alternate tiles": (np.floor(np.arange(f) / rows_per_tile).astype(int) % 2) == 0}
    for name, m in masks.items():
        say(f"    {name}: {int(m.sum())} active")
        y, idx, n_act = run_decode(layer, xd, None, ws, mask=m[None].astype(np.uint8))
        assert n_act[0] == m.sum() and np.array_equal(idx[0][:n_act[0]], np.flatnonzero(m))
        assert normwise_err(y[0], oracle.masked_ffn(Wg, Wu, Dt, x, m, "silu")) <= TOL_BF16
        y2, _, _ = run_decode(layer, xd, None, ws, mask=m[None].astype(np.uint8))
        assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


def test_balancing_declined_keeps_each_tiles_rows():
    """The path a launch takes when not all of its tiles are resident (another such call
    in flight): forced here from the host by writing "no" into the decision word of the
    workspace header before the call, so the last workgroup's "yes" finds it taken. Every
    tile then streams its own rows: y against the oracle on the library's mask within the
    fp32 bound, the same mask as the balanced call, header zero and no status afterwards."""
    w = inputs.workload(4)
    d, f, k = 8192, 6000, 0.5
    raw, dev, host = swiglu_layer_dev(w, 0, d=d, f=f)
    Wg, Wu, Dt = host["w_gate"], host["w_up"], host["w_down_t"]
    layer = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"])
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, 1))
    xcal = to_f64(inputs.tokens(w, w.n_cal, inputs.STREAM_CAL, d=d), w.dtype)
    t = float(oracle.calibrate_cats(Wg, xcal, k)[1])
    x_raw = inputs.tokens(w, 2, inputs.STREAM_DECODE, d=d)
    decision = B.SFN_WORKSPACE_STATUS_OFFSET + 4  # the word after the status word
    for j in range(2):
        xd = to_dev(x_raw[j:j + 1], w.dtype)
        yb, ib, nb_ = run_decode(layer, xd, t, ws)  # balanced (nothing overlaps)
        ws[decision:decision + 4] = torch.tensor([2, 0, 0, 0], dtype=torch.uint8, device="cuda")
        y, idx, n_act = run_decode(layer, xd, t, ws)  # checks the header is zero again
        assert B.workspace_status(ws) == 0
        gm = mask_from_idx(idx[0], n_act[0], f)
        assert n_act[0] == nb_[0] and np.array_equal(idx[0][:n_act[0]], ib[0][:nb_[0]])
        x = to_f64(x_raw, w.dtype)[j]
        e = normwise_err(y[0], oracle.masked_ffn(Wg, Wu, Dt, x, gm, "silu"))
        assert e <= min(TOL_BF16, fp32_output_bound(Wg, Wu, Dt, x, gm, "silu")), e
        say(f"    token {j}: {n_act[0]} active, error {e:.2e}, "
            f"{'bitwise equal to' if np.array_equal(y.view(np.uint32), yb.view(np.uint32)) else 'differs from'} "
            f"the balanced call")


def test_qwen2_7b_layer():
    """SparseQwen2-7B FFN shape: d 3584 is 448 16-byte chunks, not a power of two, so
    part of each row's threads hold no chunk."""
    w = inputs.workload(5)
    _case(w, w.d, w.f, 0.5, 2)


@pytest.mark.parametrize("k,n_tok", [(0.5, 8), (0.6, 4)])
def test_batch4_union_llama3_8b_layer(k, n_tok):
    """The Llama-3-8B layer at both of its sparsities, in batches of four."""
    w = inputs.workload(2)
    layer, ws, dev, host, t = _case(w, w.d, w.f, k, n_tok, batch=4)
    # each token of the batch equals its single-token run (same mask, same output up to
    # the fixed reduction order of the split-k partials)
    xs_raw = inputs.tokens(w, 4, inputs.STREAM_DECODE)
    y4, idx4, n4 = run_decode(layer, to_dev(xs_raw, w.dtype), t, ws)
    ws1 = B.workspace(B.sparse_ffn_workspace_size(layer, 1))
    for b in range(4):
        y1, idx1, n1 = run_decode(layer, to_dev(xs_raw[b:b + 1], w.dtype), t, ws1)
        # the batch gate runs on matrix cores, the single-token gate on vector units:
        # their sums differ by rounding, so a neuron within rounding of t may flip
        m1, m4 = mask_from_idx(idx1[0], n1[0], w.f), mask_from_idx(idx4[b], n4[b], w.f)
        assert (m1 != m4).sum() <= 2
        if np.array_equal(m1, m4):
            assert normwise_err(y4[b], y1[0]) <= 1e-5


def test_batch_shares_far_from_their_tiles():
    """Batches whose union rows sit far from an even spread over the gate tiles (mask
    override), so the up/down workgroups' shares of the concatenated list lie outside the
    list slots they prefetch around their tiles and take the fallback loads: every row of
    the first third, of the last third, each token its own quarter, a sparse comb. Per
    token: the index list equals the mask, y against the oracle on that mask, bitwise
    equal on a second call."""
    w = inputs.workload(2)
    d, f, nb = w.d, w.f, 4
    raw, dev, host = swiglu_layer_dev(w, 0, d=d, f=f)
    Wg, Wu, Dt = host["w_gate"], host["w_up"], host["w_down_t"]
    layer = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"])
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, nb))
    xs_raw = inputs.tokens(w, nb, inputs.STREAM_DECODE, d=d)
    xs = to_f64(xs_raw, w.dtype)
    xd = to_dev(xs_raw, w.dtype)
    rows = np.arange(f)
    masks = {"first third": np.repeat((rows < f // 3)[None], nb, 0),
             "last third": np.repeat((rows >= 2 * f // 3)[None], nb, 0),
             "own quarter": np.stack([(rows >= b * f // 4) & (rows < (b + 1) * f // 4) for b in range(nb)]),
             "comb": np.repeat((rows % 97 == 5)[None], nb, 0)}
    for name, m in masks.items():
        say(f"    {name}: union {int(m.any(0).sum())} rows")
        y, idx, n_act = run_decode(layer, xd, None, ws, mask=m.astype(np.uint8))
        for b in range(nb):
            assert n_act[b] == m[b].sum() and np.array_equal(idx[b][:n_act[b]], np.flatnonzero(m[b]))
            ref = oracle.masked_ffn(Wg, Wu, Dt, xs[b], m[b], "silu")
            assert normwise_err(y[b], ref) <= min(TOL_BF16, fp32_output_bound(Wg, Wu, Dt, xs[b], m[b]))
        y2, _, _ = run_decode(layer, xd, None, ws, mask=m.astype(np.uint8))
        assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("batch", [2, 3])
def test_partial_batches(batch):
    w = inputs.workload(1)
    _case(w, 1024, 2500, 0.5, 6, batch=batch)


@pytest.mark.parametrize("d,f,batch", [(1024, 777, 3), (520, 2000, 4), (8192, 2000, 2), (2048, 16, 4),
                                       (128, 17, 2), (4096, 16384, 4)])
def test_ragged_batches(d, f, batch):
    """Batches on the matrix-core gate, whose tile count is rounded up to a multiple of
    256: tiles of a few rows (f 777, 2000), mostly empty tiles (f 16, 17: one row or none
    per tile), a K range that ends inside a stage (d 520), several stages (d 8192), and the
    largest f it takes (16384 rows, 1024 tiles of 16)."""
    w = inputs.workload(1)
    _case(w, d, f, 0.5, 2 * batch, batch=batch)


def test_density_one_is_dense_and_relu_zero_is_dense():
    w = inputs.workload(1)
    d, f = 1024, 3000
    raw, dev, host = swiglu_layer_dev(w, 3, d=d, f=f)
    Wg, Wu, Dt = host["w_gate"], host["w_up"], host["w_down_t"]
    xs_raw = inputs.tokens(w, 2, inputs.STREAM_DECODE, d=d)
    xs = to_f64(xs_raw, w.dtype)
    for act, t in (("silu", -1.0), ("relu", 0.0)):
        say(f"[decode] dense equivalence act={act} t={t}")
        layer = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"],
                           act=B.SFN_ACT_SILU if act == "silu" else B.SFN_ACT_RELU)
        ws = B.workspace(B.sparse_ffn_workspace_size(layer, 2))
        y, idx, n_act = run_decode(layer, to_dev(xs_raw, w.dtype), t, ws)
        for b in range(2):
            yd = oracle.dense_ffn(Wg, Wu, Dt, xs[b], act)
            assert normwise_err(y[b], yd) <= TOL_BF16
            if act == "silu":
                assert n_act[b] == f
            else:
                g, _ = oracle.gate_up(Wg, Wu, xs[b])
                sig = np.sqrt((Wg * Wg).sum(1)) * np.sqrt((xs[b] ** 2).mean())
                check_mask(mask_from_idx(idx[b], n_act[b], f), g > 0, g, 0.0, abs_band=1e-3 * sig)


def test_mask_only_and_empty_mask_and_determinism():
    w = inputs.workload(1)
    d, f = 4096, 11008
    raw, dev, host = swiglu_layer_dev(w, 0, d=d, f=f)
    layer = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"])
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, 1))
    x_raw = inputs.tokens(w, 1, inputs.STREAM_DECODE)
    xd = to_dev(x_raw, w.dtype)
    say("[decode] mask-only mode")
    _, idx_m, n_m = run_decode(layer, xd, 0.265, ws, want_y=False)
    y_a, idx_a, n_a = run_decode(layer, xd, 0.265, ws)
    assert n_m[0] == n_a[0] and np.array_equal(idx_m[0][:n_m[0]], idx_a[0][:n_a[0]])
    say("[decode] determinism")
    for _ in range(3):
        y_b, idx_b, n_b = run_decode(layer, xd, 0.265, ws)
        assert np.array_equal(y_a.view(np.uint32), y_b.view(np.uint32))
        assert np.array_equal(idx_a, idx_b) and np.array_equal(n_a, n_b)
    say("[decode] empty mask")
    y0, _, n0 = run_decode(layer, xd, 0.265, ws, mask=np.zeros((1, f), np.uint8))
    assert n0[0] == 0 and np.all(y0 == 0.0)
    say("[decode] threshold above every score")
    y1, _, n1 = run_decode(layer, xd, 1e30, ws)
    assert n1[0] == 0 and np.all(y1 == 0.0)


@pytest.mark.parametrize("d", [2048, 8192])
def test_candidate_mode_reglu(d):
    """Gate evaluated on a candidate list only (ReLU, bias): oracle reglu_sequential. At
    d 8192 the tiles (shares of the candidate list) balance their up/down rows."""
    w = inputs.workload(3)
    f = 5000
    raw = inputs.reglu_layer(w, 0, d=d, f=f)
    Wg, Wu, Dt = (to_f64(raw[k], "bf16") for k in ("w_gate", "w_up", "w_down_t"))
    b = raw["b_gate"].astype(np.float64)
    layer = B.FFNLayer(to_dev(raw["w_gate"], "bf16"), to_dev(raw["w_up"], "bf16"), to_dev(raw["w_down_t"], "bf16"),
                       b_gate=torch.from_numpy(raw["b_gate"]).cuda(), act=B.SFN_ACT_RELU)
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, 1))
    xs_raw = inputs.tokens(w, 3, inputs.STREAM_DECODE, d=d)
    xs = to_f64(xs_raw, "bf16")
    rng = np.random.default_rng(5)
    for j, dens in enumerate((0.25, 0.0, 1.0)):
        say(f"[decode] candidate mode density {dens}")
        cand = np.flatnonzero(rng.random(f) < dens).astype(np.int32)
        cm = np.zeros(f, bool)
        cm[cand] = True
        cand_d = torch.from_numpy(np.concatenate([cand, np.zeros(f - len(cand), np.int32)])).cuda()
        n_cand = torch.tensor([len(cand)], dtype=torch.int32, device="cuda")
        y, idx, n_act = run_decode(layer, to_dev(xs_raw[j:j + 1], "bf16"), 0.0, ws, cand=cand_d, n_cand=n_cand)
        active, g, yo = oracle.reglu_sequential(Wg, Wu, Dt, xs[j], cm, b)
        sig = np.sqrt((Wg * Wg).sum(1)) * np.sqrt((xs[j] ** 2).mean())
        gm = mask_from_idx(idx[0], n_act[0], f)
        check_mask(gm, active, g, 0.0, abs_band=1e-3 * sig)
        assert not (gm & ~cm).any(), "active outside the candidate set"
        _, _, y_own = oracle.reglu_sequential(Wg, Wu, Dt, xs[j], gm, b)
        if np.abs(y_own).max() > 0:
            assert normwise_err(y[0], y_own) <= TOL_BF16
        else:
            assert np.all(y[0] == 0.0)


@pytest.mark.parametrize("d", [2048, 8192])
def test_candidate_entries_and_count_are_clamped(d):
    """Candidate lists are device data the host never sees, so the kernels clamp them:
    the count into [0, f] and every entry into [0, f). A list of every row whose first
    entry is -3 and last is f + 7, with a count of f + 50, is therefore every row once:
    candidate mode and the one-pass parallel call both give the dense ReGLU FFN."""
    w = inputs.workload(3)
    f = 3000
    raw = inputs.reglu_layer(w, 1, d=d, f=f)
    Wg, Wu, Dt = (to_f64(raw[k], "bf16") for k in ("w_gate", "w_up", "w_down_t"))
    b = raw["b_gate"].astype(np.float64)
    layer = B.FFNLayer(to_dev(raw["w_gate"], "bf16"), to_dev(raw["w_up"], "bf16"), to_dev(raw["w_down_t"], "bf16"),
                       b_gate=torch.from_numpy(raw["b_gate"]).cuda(), act=B.SFN_ACT_RELU)
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, 1))
    xs_raw = inputs.tokens(w, 1, inputs.STREAM_DECODE, d=d)
    x = to_f64(xs_raw, "bf16")[0]
    say(f"[decode] clamped candidate list d={d} f={f}")
    lst = np.arange(f, dtype=np.int32)
    lst[0], lst[-1] = -3, f + 7
    cand_d = torch.from_numpy(lst).cuda()
    n_cand = torch.tensor([f + 50], dtype=torch.int32, device="cuda")
    every = np.ones(f, bool)
    active, g, yo = oracle.reglu_sequential(Wg, Wu, Dt, x, every, b)
    assert np.allclose(yo, oracle.dense_ffn(Wg, Wu, Dt, x, "relu", b))
    sig = np.sqrt((Wg * Wg).sum(1)) * np.sqrt((x ** 2).mean())
    y, idx, n_act = run_decode(layer, to_dev(xs_raw, "bf16"), 0.0, ws, cand=cand_d, n_cand=n_cand)
    gm = mask_from_idx(idx[0], n_act[0], f)
    check_mask(gm, active, g, 0.0, abs_band=1e-3 * sig)
    _, _, y_own = oracle.reglu_sequential(Wg, Wu, Dt, x, gm, b)
    assert normwise_err(y[0], y_own) <= TOL_BF16
    yp = torch.full((d,), float("nan"), dtype=torch.float32, device="cuda")
    B.sparse_ffn_decode_parallel(layer, to_dev(xs_raw[0], "bf16"), cand_d, n_cand, ws, yp)
    torch.cuda.synchronize()
    assert _header_clear(ws)
    assert normwise_err(yp.cpu().numpy(), yo) <= TOL_BF16


@pytest.mark.parametrize("d,want_y", [(1024, True), (1024, False), (8192, True)])
def test_empty_candidate_list(d, want_y):
    """n_cand = 0 leaves every gate tile without rows (regression: a tile with no rows
    once fetched its bias through a row index read from LDS it had never written). The
    call must produce y = 0 and no active rows, with a bias present to be fetched: the
    one-token loop (d 1024), the gate alone (no y) and the balanced path (d 8192)."""
    w = inputs.workload(3)
    f = 3000
    raw = inputs.reglu_layer(w, 0, d=d, f=f)
    layer = B.FFNLayer(to_dev(raw["w_gate"], "bf16"), to_dev(raw["w_up"], "bf16"), to_dev(raw["w_down_t"], "bf16"),
                       b_gate=torch.from_numpy(raw["b_gate"]).cuda(), act=B.SFN_ACT_RELU)
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, 1))
    xd = to_dev(inputs.tokens(w, 1, inputs.STREAM_DECODE, d=d), "bf16")
    cand = torch.zeros(f, dtype=torch.int32, device="cuda")
    n_cand = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        y, idx, n_act = run_decode(layer, xd, 0.0, ws, want_y=want_y, cand=cand, n_cand=n_cand)
        assert np.all(n_act == 0)
        if want_y:
            assert np.all(y == 0.0)


def test_one_workspace_shared_by_every_call():
    """calibrate -> decode -> dense chunk -> predictor -> decode -> calibrate -> decode on a
    single workspace: each call must leave the reserved header as it found it
    (regression: the calibration state once overlapped a decode counter)."""
    w = inputs.workload(1)
    d, f, n_cal = 2048, 3000, 64
    raw, dev, host = swiglu_layer_dev(w, 0, d=d, f=f)
    Wg, Wu, Dt = host["w_gate"], host["w_up"], host["w_down_t"]
    layer = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"])
    Q, L = oracle.svd_factors(Wg, 64)
    Qb, Lb = inputs.f32_to_bf16_bits(Q), inputs.f32_to_bf16_bits(L)
    pred = B.SVDPredictor(to_dev(Qb, "bf16"), to_dev(Lb, "bf16"), torch.zeros(f, dtype=torch.float32, device="cuda"))
    ws = B.workspace(max(B.sparse_ffn_workspace_size(layer, n_cal), B.svd_predict_workspace_size(pred)))
    xcal_raw = inputs.tokens(w, n_cal, inputs.STREAM_CAL, d=d)
    xs_raw = inputs.tokens(w, 3, inputs.STREAM_DECODE, d=d)
    xs = to_f64(xs_raw, "bf16")
    t_dev = torch.empty(1, dtype=torch.float32, device="cuda")

    def decode_check(j):
        y = torch.empty((1, d), dtype=torch.float32, device="cuda")
        idx = torch.empty((1, f), dtype=torch.int32, device="cuda")
        n_act = torch.empty(1, dtype=torch.int32, device="cuda")
        B.sparse_ffn_decode(layer, to_dev(xs_raw[j:j + 1], "bf16"), t_dev, ws, y=y, active_idx=idx, n_active=n_act)
        torch.cuda.synchronize()
        assert _header_clear(ws)
        t = float(t_dev.item())
        gm = mask_from_idx(idx.cpu().numpy()[0], int(n_act.item()), f)
        om, oa, _ = oracle.cats_decode(Wg, Wu, Dt, xs[j][None], t)
        check_mask(gm, om[0], np.abs(oa[0]), t)
        assert normwise_err(y.cpu().numpy()[0], oracle.masked_ffn(Wg, Wu, Dt, xs[j], gm)) <= TOL_BF16

    say("[shared ws] calibrate, decode")
    B.sparse_ffn_calibrate(layer, to_dev(xcal_raw, "bf16"), 0.5, t_dev, ws)
    decode_check(0)
    say("[shared ws] dense chunk")
    yc = torch.empty((3, d), dtype=torch.float32, device="cuda")
    for _ in range(2):
        B.ffn_dense_chunk(layer, to_dev(xs_raw, "bf16"), yc, ws)
        torch.cuda.synchronize()
        Yo = oracle.dense_chunk(Wg, Wu, Dt, xs)
        for j in range(3):
            assert normwise_err(yc.cpu().numpy()[j], Yo[j]) <= TOL_BF16
    say("[shared ws] predictor, decode")
    cand = torch.empty(f, dtype=torch.int32, device="cuda")
    n_cand = torch.empty(1, dtype=torch.int32, device="cuda")
    B.svd_predict(pred, to_dev(xs_raw[1], "bf16"), cand, n_cand, ws)
    decode_check(1)
    say("[shared ws] calibrate again, decode")
    B.sparse_ffn_calibrate(layer, to_dev(xcal_raw, "bf16"), 0.7, t_dev, ws)
    decode_check(2)


@pytest.mark.parametrize("d,f,batch", [(16384, 600, 1), (16384, 600, 4), (64, 262144, 1), (64, 262144, 3)])
def test_limits(d, f, batch):
    """The largest rows (d 16384: four 16-byte chunks per thread) and the most neurons
    (f 262144: 1024 tiles of 256 rows, the most a launch takes)."""
    w = inputs.workload(1)
    _case(w, d, f, 0.5, batch, batch=batch)


def _same_as_sequential(together, seq, d):
    """Overlapping calls give the sequential results bit for bit, except one-token calls
    on rows wider than 8 KB (d > 4096 in bf16): a call whose tiles are not all resident at
    once keeps its rows unbalanced and sums them in another order, so there the results
    agree to fp32 rounding."""
    assert not torch.isnan(together).any()
    if d <= 4096:
        assert torch.equal(together.view(torch.int32), seq.view(torch.int32))
    else:
        err = (together - seq).abs().amax(dim=-1) / seq.abs().amax(dim=-1)
        assert float(err.max()) <= 1e-5, float(err.max())


def test_concurrent_streams_with_separate_workspaces():
    """Calls on two streams at once, each with its own workspace, give the results of the
    same calls one after another: the library keeps no state outside the caller's buffers
    (one-token calls at 8 KB rows, four-token batches, a calibration, and one-token calls
    at 16 KB rows, whose tiles balance through their own workspace's header when all of
    them are resident)."""
    w = inputs.workload(1)
    cases = [(4096, 11008, 1), (4096, 14336, 4), (8192, 6000, 1)]
    for d, f, nb in cases:
        say(f"[streams] d={d} f={f} B={nb}")
        raw, dev, host = swiglu_layer_dev(w, 0, d=d, f=f)
        layer = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"])
        n_tok = 6
        xs = to_dev(inputs.tokens(w, n_tok * nb, inputs.STREAM_DECODE, d=d), "bf16").view(n_tok, nb, d)
        xcal = to_dev(inputs.tokens(w, 64, inputs.STREAM_CAL, d=d), "bf16")
        wss = [B.workspace(B.sparse_ffn_workspace_size(layer, 64)) for _ in range(2)]
        t = torch.empty(2, dtype=torch.float32, device="cuda")
        ys = torch.full((2, n_tok, nb, d), float("nan"), dtype=torch.float32, device="cuda")
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
        torch.cuda.synchronize()

        def work(i, st):
            B.sparse_ffn_calibrate(layer, xcal, 0.5 + 0.2 * i, t[i:i + 1], wss[i], stream=st)
            for j in range(n_tok):
                B.sparse_ffn_decode(layer, xs[j], t[i:i + 1], wss[i], y=ys[i, j], stream=st)

        for i, st in enumerate(streams):  # both streams in flight together
            with torch.cuda.stream(st):
                work(i, st)
        torch.cuda.synchronize()
        together = ys.clone()
        ys.fill_(float("nan"))
        for i in range(2):  # the same calls one after another on the current stream
            work(i, torch.cuda.current_stream())
            torch.cuda.synchronize()
        _same_as_sequential(together, ys, d)
        for ws in wss:
            assert _header_clear(ws)


def test_host_threads_with_separate_streams():
    """Two host threads submit calls at the same time, each on its own stream with its own
    workspace (the binding releases the interpreter lock inside each call, so the library's
    host code runs concurrently, including its per-device caches): the results of the same
    calls made one after another. At d 8192 two balanced one-token calls can overlap on the
    device; a call whose tiles are not all resident, because the other call holds compute
    units, does not wait for them but keeps its rows unbalanced (results equal to fp32
    rounding, never NaN)."""
    import threading
    w = inputs.workload(1)
    for d, f, nb in [(4096, 11008, 1), (8192, 6000, 1), (4096, 14336, 4)]:
        say(f"[threads] d={d} f={f} B={nb}")
        raw, dev, host = swiglu_layer_dev(w, 1, d=d, f=f)
        layer = B.FFNLayer(dev["w_gate"], dev["w_up"], dev["w_down_t"])
        n_tok = 8
        xs = to_dev(inputs.tokens(w, n_tok * nb, inputs.STREAM_DECODE, d=d), "bf16").view(n_tok, nb, d)
        xcal = to_dev(inputs.tokens(w, 64, inputs.STREAM_CAL, d=d), "bf16")
        wss = [B.workspace(B.sparse_ffn_workspace_size(layer, 64)) for _ in range(2)]
        t = torch.empty(2, dtype=torch.float32, device="cuda")
        ys = torch.full((2, n_tok, nb, d), float("nan"), dtype=torch.float32, device="cuda")
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]  # default priority
        torch.cuda.synchronize()
        start = threading.Barrier(2)
        errors = []

        def work(i, st, wait):
            try:
                if wait:
                    start.wait(timeout=30)
                with torch.cuda.stream(st):
                    B.sparse_ffn_calibrate(layer, xcal, 0.5 + 0.2 * i, t[i:i + 1], wss[i], stream=st)
                    for j in range(n_tok):
                        B.sparse_ffn_decode(layer, xs[j], t[i:i + 1], wss[i], y=ys[i, j], stream=st)
                st.synchronize()
            except Exception as e:  # reported by the main thread
                errors.append(e)

        threads = [threading.Thread(target=work, args=(i, streams[i], True)) for i in range(2)]
        for th in threads:
            th.start()
        for th in threads:
            th.join(timeout=60)
        assert not errors, errors
        assert not any(th.is_alive() for th in threads)
        torch.cuda.synchronize()
        together = ys.clone()
        ys.fill_(float("nan"))
        for i in range(2):  # one after another, on this thread
            work(i, torch.cuda.current_stream(), False)
            torch.cuda.synchronize()
        assert not errors, errors
        _same_as_sequential(together, ys, d)
        for ws in wss:
            assert _header_clear(ws)
