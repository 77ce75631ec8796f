#!/usr/bin/env python3
"""Sparse-FFN decode benchmark on one MI355X.

Workload: the Llama-2-7B-shaped SwiGLU FFN stack -- 32 layers, hidden 4096,
intermediate 11008, bf16 weights ~ N(0, 0.02^2) generated on the device from fixed
seeds, batch 1, every layer of every token fed its own x ~ N(0, I) (bf16). CATS
thresholds are calibrated per layer by the library (256 calibration tokens) for the
headline sparsity (50%) and for the sweep points (70/80/90%).

A step is one decode token through all 32 layers (32 sparse_ffn_decode calls; each call
is two kernels: gate with each tile's up/down, then the reduce). After W untimed warm-up steps, K steps are
timed with HIP events on the stream the kernels run on (graph mode: one captured graph
per token, replayed back to back). The JSON line on stdout carries:
  value      decode tokens/s at the headline sparsity (inputs resident in HBM)
  roofline   one sparse_ffn_decode call: algorithmic bytes per call (all gate rows, the
             active up and down rows, x and y) over the average call duration in the
             timed region, against the 8 TB/s HBM peak; `stages` splits the call into
             the gate (the gate kernel timed alone, from calls that request no output)
             and the rest; `traffic` is the HBM bytes per call from the committed rocprofv3
             counter summary, when that summary was taken on the current kernel source
  cpu_baseline  the CPU oracle (dense FFN then mask, numpy float64) timed on a bounded
             sample of layers and tokens of the same workload on this host
  dense_path the same stack through the library's dense path (ffn_dense_chunk, n = 1)
  sweep      tokens/s, density and GB/s at the other sparsities
Progress goes to stderr.

Profiling helpers (no GPU needed): --summarize-trace DIR turns a rocprofv3
--kernel-trace --stats CSV output into a markdown table; --summarize-traffic FETCH_DIR
WRITE_DIR turns two --pmc CSV outputs (FETCH_SIZE, then WRITE_SIZE) of a
`--copy-probe` run into HBM bytes per decode call, scaled by what the counters read for
the probe's plain copy of known size.
"""

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_llama2_7b_k50_traffic.json")
KERNEL_SOURCES = ["contextual_activation_sparsity_amd/csrc/decode.hip",
                  "contextual_activation_sparsity_amd/csrc/device_common.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash():
    """Hash of the decode kernels' code: the sources with comments and blank space
    removed, so that a change to a comment does not invalidate the counter summary."""
    import re
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=32)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--sparsity", type=float, default=0.5)
    ap.add_argument("--sweep", type=str, default="0.7,0.8,0.9")
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--mode", choices=("graph", "eager"), default="graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other workloads (batch 4, SVD pipeline, 70B-shape decode and 16-token chunk)")
    ap.add_argument("--svd-layers", type=int, default=32, help="layers of the timed SVD stacks")
    ap.add_argument("--svd-prepared", type=int, default=4,
                    help="distinct prepared ReGLU layers (factors, thresholds) the SVD stacks copy")
    ap.add_argument("--svd-prep-host", action="store_true",
                    help="compute the SVD legs' factors on the host in float64 instead of on the device")
    ap.add_argument("--legs", default=",".join(EXTRA_LEGS),
                    help="comma list of the other workloads to run: " + ", ".join(EXTRA_LEGS))
    ap.add_argument("--no-table4", action="store_true",
                    help="skip the fixed-sparsity protocol (random candidate subsets on every layer, three shapes)")
    ap.add_argument("--t4-shapes", default="0,1,2",
                    help="comma list of the fixed-sparsity protocol's shapes to run (0: 4096/11008, 1: 4096/14336, "
                         "2: 3584/18944)")
    ap.add_argument("--t4-sparsities", default="0.2,0.5,0.8,0.95")
    ap.add_argument("--no-quality", action="store_true",
                    help="skip the predictor-quality diagnostics (ROC AUC and recall against rank and s)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="before the stack, copy a MIB-MiB buffer three times (counter scaling)")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-kernel-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--command", default="", help="profiling command recorded in a summary")
    return ap.parse_args()


DECODE_KERNELS = ("decode_gate_local_kernel", "decode_gate_kernel", "decode_updown_kernel", "decode_reduce_kernel")
# the kernels of one batch-1 decode call (the gate kernel alone runs in the gate-only timing)
CALL_KERNELS = ("decode_gate_local_kernel", "decode_reduce_kernel")
COPY_KERNEL = "copy_kernel"


def _csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for fn in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(fn, newline="") as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no *{suffix} under {d}")
    return rows


def _short(name, keep_args=False):
    if keep_args:
        import re
        m = re.search(r"(\w+_kernel)(<[^>]*>)?\(", name.replace("(anonymous namespace)::", ""))
        if m and "sfn::" in name:
            return m.group(1) + (m.group(2) or "").replace(" ", "")
    for k in DECODE_KERNELS + ("chunk_stage1_kernel", "chunk_stage2_kernel", "chunk_reduce_kernel",
                               "score_mfma_kernel", "score_kernel", "hist_kernel", "pick_kernel", "set_kernel",
                               "svd_z_kernel", "svd_p_kernel"):
        if k in name:
            return k
    if "elementwise_kernel" in name and "neg" in name.lower():
        return COPY_KERNEL
    return name[:60]


def summarize_trace(d, command):
    """Markdown table of the library's kernels from a rocprofv3 --kernel-trace CSV output:
    dispatches grouped by kernel and grid size (one group per shape), then torch's own
    kernels (weight generation and the like) in one line."""
    import statistics
    rows = _csv_rows(d, "kernel_trace.csv")
    groups, other_n, other_ns = {}, 0, 0.0
    for r in rows:
        name = r["Kernel_Name"]
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if "sfn::" not in name:
            other_n += 1
            other_ns += dur
            continue
        grid = int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        wgs = grid // max(1, int(r["Workgroup_Size_X"]) * int(r["Workgroup_Size_Y"]) * int(r["Workgroup_Size_Z"]))
        groups.setdefault((_short(name, keep_args=True), wgs, int(r["Workgroup_Size_X"])), []).append(dur)
    out = ["# rocprofv3 kernel trace summary", "", "Command:", "", "```", command or "(not recorded)", "```", "",
           "Template arguments of the decode kernels: <weight dtype (1 bf16, 0 fp32), tokens held (1 or 4), "
           "16-byte chunks per thread, threads per row, rows per thread per step>.", "",
           "| kernel | workgroups x threads | dispatches | average us | median us | min us | max us |",
           "|---|---|---|---|---|---|---|"]
    for (k, wgs, wgsz), v in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| `{k}` | {wgs} x {wgsz} | {len(v)} | {statistics.mean(v):.2f} | {statistics.median(v):.2f} | "
                   f"{min(v):.2f} | {max(v):.2f} |")
    out.append(f"| (torch kernels: input generation, copies) | | {other_n} | {other_ns / max(1, other_n):.2f} | | | |")
    print("\n".join(out))


def summarize_traffic(fetch_dir, write_dir, probe_bytes):
    """Median FETCH_SIZE / WRITE_SIZE bytes per dispatch of each kernel (the counters are
    in KiB), and what they read for the probe's copy of probe_bytes bytes."""
    import statistics
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = {}
        for r in _csv_rows(d, "counter_collection.csv"):
            if r.get("Counter_Name") != counter:
                continue
            per.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]) * 1024.0)
        copies = per.get(COPY_KERNEL)
        if not copies:
            raise SystemExit(f"{counter}: the copy probe's kernel is missing")
        res[counter] = {"per_kernel_bytes": {k: statistics.median(v) for k, v in per.items()},
                        "copy_probe_bytes_counted": statistics.median(copies), "copy_probe_bytes": probe_bytes}
    return res


class Stack:
    """Device weights, thresholds and per-token inputs of the benchmark stack."""

    def __init__(self, B, inputs, torch, n_layers, n_tokens):
        self.B, self.torch = B, torch
        w = inputs.workload(1)
        self.w, self.d, self.f, self.L = w, w.d, w.f, n_layers
        dev = "cuda"
        self.layers = []
        for l in range(n_layers):
            wg = inputs.torch_gaussian_bf16((w.f, w.d), w.w_std, inputs.seed(w.index, l, inputs.T_GATE), dev)
            wu = inputs.torch_gaussian_bf16((w.f, w.d), w.w_std, inputs.seed(w.index, l, inputs.T_UP), dev)
            wd = inputs.torch_gaussian_bf16((w.f, w.d), w.w_std, inputs.seed(w.index, l, inputs.T_DOWN), dev)
            self.layers.append(B.FFNLayer(wg, wu, wd))
        g = torch.Generator(device=dev)
        g.manual_seed(1_000_000 * w.index + inputs.STREAM_DECODE)
        self.X = torch.randn((n_tokens, n_layers, w.d), generator=g, device=dev).to(torch.bfloat16)
        xcal = inputs.tokens(w, w.n_cal, inputs.STREAM_CAL)
        import numpy as np
        self.xcal = torch.from_numpy(xcal.view(np.int16)).view(torch.bfloat16).to(dev)
        self.ws = B.workspace(B.sparse_ffn_workspace_size(self.layers[0], w.n_cal))
        self.Y = torch.zeros((n_layers, w.d), dtype=torch.float32, device=dev)
        self.n_act = torch.zeros((n_tokens, n_layers), dtype=torch.int32, device=dev)
        self.thr = {}
        self.lib = B.raw()

    def calibrate(self, k):
        t = self.torch.zeros(self.L, dtype=self.torch.float32, device="cuda")
        for l, layer in enumerate(self.layers):
            self.B.sparse_ffn_calibrate(layer, self.xcal, k, t[l:l + 1], self.ws)
        self.torch.cuda.synchronize()
        self.thr[k] = t
        return t

    def decode_args(self, tok, k, stream, with_counts=False):
        """Raw ctypes argument tuples of one step (token `tok`, sparsity k)."""
        t = self.thr[k]
        wsb = self.ws.numel()
        out = []
        for l, layer in enumerate(self.layers):
            out.append((ctypes.byref(layer.c), self.X[tok, l].data_ptr(), 1, t[l:l + 1].data_ptr(), None, None, None,
                        self.Y[l].data_ptr(), None,
                        self.n_act[tok, l:l + 1].data_ptr() if with_counts else None,
                        self.ws.data_ptr(), wsb, stream))
        return out

    def dense_args(self, tok, stream):
        wsb = self.ws.numel()
        return [(ctypes.byref(layer.c), self.X[tok, l].data_ptr(), 1, self.Y[l].data_ptr(), self.ws.data_ptr(), wsb,
                 stream) for l, layer in enumerate(self.layers)]


def run_calls(fn, calls):
    for a in calls:
        st = fn(*a)
        if st != 0:
            raise RuntimeError(f"library call failed with status {st}")


def warm_graphs(torch, graphs):
    """Replay every captured graph once, untimed, so that the timed pass measures steady
    replays: a graph's first replay also uploads it to the device (several microseconds
    per graph, which would be charged to the few calls of a short graph). The replays
    run the same work again on the same inputs; with stacks far larger than the caches
    no weights are left in them for the timed pass."""
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()


def time_steps(torch, fn, step_args, mode):
    """Time len(step_args) steps. Graph mode captures one graph per step (each token has
    its own inputs) and replays them back to back."""
    stream = torch.cuda.current_stream()
    if mode == "graph":
        graphs = []
        cap = torch.cuda.Stream()
        for calls in step_args:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                run_calls(fn, [a[:-1] + (cap.cuda_stream,) for a in calls])
            graphs.append(g)
        warm_graphs(torch, graphs)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for g in graphs:
            g.replay()
        e1.record(stream)
    else:
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for calls in step_args:
            run_calls(fn, calls)
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def time_mixed(torch, steps, mode):
    """Like time_steps, for steps whose calls go to different library functions:
    steps = [[(fn, args_without_stream), ...], ...]. Returns ms for all steps."""
    stream = torch.cuda.current_stream()

    def run(step, st):
        for fn, a in step:
            rc = fn(*a, st)
            if rc != 0:
                raise RuntimeError(f"library call failed with status {rc}")

    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if mode == "graph":
        graphs = []
        cap = torch.cuda.Stream()
        for step in steps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                run(step, cap.cuda_stream)
            graphs.append(g)
        warm_graphs(torch, graphs)
        e0.record(stream)
        for g in graphs:
            g.replay()
        e1.record(stream)
    else:
        e0.record(stream)
        for step in steps:
            run(step, stream.cuda_stream)
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


EXTRA_LEGS = ("tiny", "b4", "b1", "70b", "chunk", "sirius", "svd")


def extras(B, inputs, torch, mode, n_steps=16, n_warm=3, legs=EXTRA_LEGS, svd_layers=32,
           svd_prepared=4, svd_prep_host=False):
    """The other workloads, each timed like the headline (graphs of per-layer calls, HIP
    events over the timed steps) on stacks of the workloads' own depth (32 independently
    seeded layers at the Llama-3-8B shape, 8 at the Llama-3-70B shape, svd_layers for the
    SVD pipelines): per-call time, algorithmic bytes and GB/s. Inputs as in the headline: on-device Gaussian weights,
    x ~ N(0, I) in bf16, thresholds from the library's own calibration. `legs` picks a
    subset (for profiling one workload at a time).

    A leg's tensors go back to torch's cache when it ends, not to the driver: for up to a
    few seconds after several GB were released (empty_cache), the next leg's batch-4 calls
    ran 4% slower (68.9 against 66.2 us at k 0.6); with the blocks reused, or after a
    pause of a few seconds, they ran at the usual rate."""
    import numpy as np
    lib = B.raw()
    dev = "cuda"
    out = {}

    def gauss(shape, std, seed):
        return inputs.torch_gaussian_bf16(shape, std, seed, dev)

    def xtok(w, shape, stream_id):
        g = torch.Generator(device=dev)
        g.manual_seed(1_000_000 * w.index + stream_id)
        return torch.randn(shape, generator=g, device=dev).to(torch.bfloat16)

    def swiglu_layers(w, d, f, nl):
        return [B.FFNLayer(gauss((f, d), w.w_std, inputs.seed(w.index, l, inputs.T_GATE)),
                           gauss((f, d), w.w_std, inputs.seed(w.index, l, inputs.T_UP)),
                           gauss((f, d), w.w_std, inputs.seed(w.index, l, inputs.T_DOWN))) for l in range(nl)]

    def calibrate(layers, w, k, ws):
        xc = torch.from_numpy(inputs.tokens(w, w.n_cal, inputs.STREAM_CAL, d=layers[0].d).view(np.int16))
        xc = xc.view(torch.bfloat16).to(dev)
        t = torch.zeros(len(layers), dtype=torch.float32, device=dev)
        for l, layer in enumerate(layers):
            B.sparse_ffn_calibrate(layer, xc, k, t[l:l + 1], ws)
        return t

    def decode_leg(name, w, d, f, batch, k, nl):
        layers = swiglu_layers(w, d, f, nl)
        ws = B.workspace(max(B.sparse_ffn_workspace_size(layers[0], max(batch, w.n_cal)),
                             B.sparse_ffn_workspace_size(layers[0], 16)))
        t = calibrate(layers, w, k, ws)
        X = xtok(w, (n_warm + n_steps, nl, batch, d), inputs.STREAM_DECODE)
        y = torch.zeros((nl, batch, d), dtype=torch.float32, device=dev)
        idx = torch.zeros((batch, f), dtype=torch.int32, device=dev)
        nact = torch.zeros(batch, dtype=torch.int32, device=dev)
        wsp, wsb = ws.data_ptr(), ws.numel()

        def call(tok, l, counts=False):
            return (lib.sparse_ffn_decode, (ctypes.byref(layers[l].c), X[tok, l].data_ptr(), batch,
                                            t[l:l + 1].data_ptr(), None, None, None, y[l].data_ptr(),
                                            idx.data_ptr() if counts else None,
                                            nact.data_ptr() if counts else None, wsp, wsb))
        # union density from the index lists of an untimed pass over the timed tokens
        union = []
        for tok in range(n_warm, n_warm + n_steps):
            for l in range(nl):
                fn, a = call(tok, l, True)
                fn(*a, torch.cuda.current_stream().cuda_stream)
                torch.cuda.synchronize()
                m = torch.zeros(f, dtype=torch.bool, device=dev)
                for b in range(batch):
                    m[idx[b, :int(nact[b].item())].long()] = True
                union.append(int(m.sum().item()))
        u = float(np.mean(union))
        time_mixed(torch, [[call(tok, l) for l in range(nl)] for tok in range(n_warm)], mode)
        ms = time_mixed(torch, [[call(tok, l) for l in range(nl)] for tok in range(n_warm, n_warm + n_steps)], mode)
        us = ms * 1e3 / (n_steps * nl)
        byts = 2.0 * f * d + 4.0 * d * u + 2.0 * batch * d + 4.0 * batch * d
        out[name] = {"d": d, "f": f, "batch": batch, "sparsity": k, "layers_timed": nl, "us_per_call": us,
                     "union_density": u / f, "algorithmic_bytes_per_call": byts,
                     "gbs": byts / (us * 1e-6) / 1e9, "tokens_per_s_timed_stack": batch / (nl * us * 1e-6),
                     "tokens_per_s_32_layers": batch / (32 * us * 1e-6)}
        log(f"  extra {name}: {us:.2f} us/call, union density {u / f:.4f}, {out[name]['gbs']:.0f} GB/s")
        del layers, ws, X, y

    def chunk_leg(w4):
        # 16-token dense verification chunk at the Llama-3-70B shape
        nl = w4.layers
        layers = swiglu_layers(w4, w4.d, w4.f, nl)
        ws = B.workspace(B.sparse_ffn_workspace_size(layers[0], 16))
        X = xtok(w4, (n_warm + n_steps, nl, 16, w4.d), inputs.STREAM_DECODE)
        Y = torch.zeros((nl, 16, w4.d), dtype=torch.float32, device=dev)
        wsp, wsb = ws.data_ptr(), ws.numel()

        def chunk(tok, l):
            return (lib.ffn_dense_chunk, (ctypes.byref(layers[l].c), X[tok, l].data_ptr(), 16, Y[l].data_ptr(), wsp, wsb))
        time_mixed(torch, [[chunk(tok, l) for l in range(nl)] for tok in range(n_warm)], mode)
        ms = time_mixed(torch, [[chunk(tok, l) for l in range(nl)] for tok in range(n_warm, n_warm + n_steps)], mode)
        us = ms * 1e3 / (n_steps * nl)
        byts = 6.0 * w4.f * w4.d + 2.0 * 16 * w4.d + 4.0 * 16 * w4.d
        out["llama3_70b_chunk16"] = {"d": w4.d, "f": w4.f, "tokens": 16, "layers_timed": nl, "us_per_call": us,
                                     "algorithmic_bytes_per_call": byts, "gbs": byts / (us * 1e-6) / 1e9,
                                     "tflops": 2.0 * 3 * w4.f * w4.d * 16 / (us * 1e-6) / 1e12,
                                     "ms_per_chunk_8_layers": 8 * us / 1e3}
        log(f"  extra chunk16: {us:.1f} us/layer, {out['llama3_70b_chunk16']['gbs']:.0f} GB/s")
        del layers, ws, X, Y


    def sirius_leg(w4):
        # Sirius correction period at the Llama-3-70B shape over an 8-layer group: 16 sparse
        # CATS steps (each token through the 8 layers), then the dense verification of the
        # same 16 tokens per layer, captured together and replayed; against full-model
        # decoding (16 one-token dense calls per layer)
        P, nlg = 16, w4.layers
        layers = swiglu_layers(w4, w4.d, w4.f, nlg)
        ws = B.workspace(max(B.sparse_ffn_workspace_size(layers[0], w4.n_cal), B.sparse_ffn_workspace_size(layers[0], P)))
        t = calibrate(layers, w4, 0.5, ws)
        n_per = 4  # one warm-up period, three timed
        X = xtok(w4, (n_per, nlg, P, w4.d), inputs.STREAM_DECODE)
        Ys = torch.zeros((nlg, P, w4.d), dtype=torch.float32, device=dev)
        Yd = torch.zeros((nlg, P, w4.d), dtype=torch.float32, device=dev)
        nact = torch.zeros((nlg, P), dtype=torch.int32, device=dev)
        wsp, wsb = ws.data_ptr(), ws.numel()

        def sparse_step(per, j, counts=False):
            return [(lib.sparse_ffn_decode, (ctypes.byref(layers[l].c), X[per, l, j].data_ptr(), 1, t[l:l + 1].data_ptr(),
                                             None, None, None, Ys[l, j].data_ptr(), None,
                                             nact[l, j:j + 1].data_ptr() if counts else None, wsp, wsb))
                    for l in range(nlg)]

        def verify(per):
            return [(lib.ffn_dense_chunk, (ctypes.byref(layers[l].c), X[per, l].data_ptr(), P, Yd[l].data_ptr(), wsp, wsb))
                    for l in range(nlg)]

        def dense_tokens(per):
            return [(lib.ffn_dense_chunk, (ctypes.byref(layers[l].c), X[per, l, j].data_ptr(), 1, Ys[l, j].data_ptr(),
                                           wsp, wsb)) for j in range(P) for l in range(nlg)]

        def period(per, counts=False):
            return [c for j in range(P) for c in sparse_step(per, j, counts)] + verify(per)
        time_mixed(torch, [period(0)], mode)
        per_ms = time_mixed(torch, [period(p) for p in range(1, n_per)], mode) / (n_per - 1)
        sparse_ms = time_mixed(torch, [[c for j in range(P) for c in sparse_step(p, j)] for p in range(1, n_per)],
                               mode) / (n_per - 1)
        verify_ms = time_mixed(torch, [verify(p) for p in range(1, n_per)], mode) / (n_per - 1)
        time_mixed(torch, [dense_tokens(0)], mode)
        dense_ms = time_mixed(torch, [dense_tokens(p) for p in range(1, n_per)], mode) / (n_per - 1)
        # outputs and active counts of the last period (untimed), then the statistics
        for fn, a in period(n_per - 1, counts=True):
            fn(*a, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        div = ((Ys - Yd).norm(dim=-1) / Yd.norm(dim=-1)).flatten().cpu().numpy()
        dens = float(nact.float().mean().item()) / w4.f
        rho = (1.0 + 2.0 * dens) / 3.0  # a CATS step's weight bytes over a dense token's
        dense_tok_bytes = 6.0 * w4.f * w4.d * nlg
        res = {"d": w4.d, "f": w4.f, "layers": nlg, "period": P, "sparsity": 0.5, "active_density": dens,
               "period_ms": per_ms, "sparse_steps_ms": sparse_ms, "verify_ms": verify_ms,
               "dense_decode_16_tokens_ms": dense_ms,
               "divergence": {"mean": float(div.mean()), "p90": float(np.quantile(div, 0.9)), "max": float(div.max())}}
        # accepted advance length: all 16, and 15.37 of 16 (the page's GSM8K figure)
        for name, aal in (("aal16", 16.0), ("aal15.37", 15.37)):
            res[name] = {"tokens_per_s": aal / (per_ms * 1e-3), "latency_vs_full": (per_ms / aal) / (dense_ms / P),
                         "effective_density": (P * rho + 1.0) / aal,
                         "effective_bytes_per_token": (P * rho + 1.0) * dense_tok_bytes / aal}
        out["llama3_70b_sirius_period16"] = res
        log(f"  extra sirius period: {per_ms:.3f} ms ({sparse_ms:.3f} sparse + {verify_ms:.3f} verify), dense 16 tokens "
            f"{dense_ms:.3f} ms, latency vs full {res['aal16']['latency_vs_full']:.3f}, divergence mean "
            f"{res['divergence']['mean']:.4f}")
        del layers, ws, X, Ys, Yd


    def svd_legs():
        # ReGLU layers with SVD predictors (factors and thresholds from the offline
        # preparation): the sequential pipeline with a rank-256 predictor (predict, then the
        # gate on the candidates and up/down where ReLU(gate) > 0) and the parallel pipeline
        # with a rank-1024 whitened predictor (predict, then gate, up and down rows of every
        # candidate in one pass)
        from contextual_activation_sparsity_amd import prepare
        w3 = inputs.workload(3)
        d, f = w3.d, w3.f
        layers, pred_seq, pred_par = [], [], []
        # calibration tokens for whitening and thresholds: 2d of them (whitening needs n >= d)
        xcal = xtok(w3, (max(w3.n_tau_cal, 2 * d), d), inputs.STREAM_TAU)
        t0 = time.perf_counter()
        for l in range(svd_prepared):
            A = torch.randn((f, w3.rank), generator=torch.Generator(device=dev).manual_seed(
                inputs.seed(3, l, inputs.T_A)), device=dev) / np.sqrt(w3.rank)
            Bm = torch.randn((w3.rank, d), generator=torch.Generator(device=dev).manual_seed(
                inputs.seed(3, l, inputs.T_B)), device=dev) * w3.w_std
            noise = torch.randn((f, d), generator=torch.Generator(device=dev).manual_seed(
                inputs.seed(3, l, inputs.T_NOISE)), device=dev) * w3.w_std
            wg = (A @ Bm + 0.1 * noise).to(torch.bfloat16)
            del A, Bm, noise
            bias = (-1.2815516 * wg.float().norm(dim=1)).contiguous()
            gates = xcal.float() @ wg.float().t() + bias
            for preds, r, whiten in ((pred_seq, 256, False), (pred_par, 1024, True)):
                if svd_prep_host:  # float64 on the host (the device SVD is the other route)
                    q, lf = (t.to(dev) for t in prepare.svd_factors(wg.cpu(), r, x_cal=xcal.cpu() if whiten else None))
                else:
                    q, lf = prepare.svd_factors(wg, r, x_cal=xcal if whiten else None)
                tau = prepare.calibrate_tau(prepare.predictions(q, lf, xcal.float(), bias), gates, w3.s)
                preds.append(B.SVDPredictor(q, lf, tau, b=bias))
                torch.cuda.synchronize()
                log(f"  layer {l}: rank-{r} {'whitened ' if whiten else ''}factors and thresholds at "
                    f"{time.perf_counter() - t0:.1f} s")
            del gates
            layers.append(B.FFNLayer(wg, gauss((f, d), w3.w_std, inputs.seed(3, l, inputs.T_UP)),
                                     gauss((f, d), w3.w_std, inputs.seed(3, l, inputs.T_DOWN)), b_gate=bias,
                                     act=B.SFN_ACT_RELU))
        torch.cuda.synchronize()
        log(f"  svd factors and thresholds for {svd_prepared} layers in {time.perf_counter() - t0:.1f} s")
        # the timed stack: svd_layers layers, layer l a copy of prepared layer l % svd_prepared
        # in memory of its own, so the working set (about 10 GB of weights and factors over
        # 32 layers) is streamed from HBM on every token, as 32 distinct layers would be;
        # preparing each layer separately would add seconds of SVD per layer and change
        # neither the bytes nor the densities
        def copy_layer(src):
            return B.FFNLayer(src.w_gate.clone(), src.w_up.clone(), src.w_down_t.clone(), b_gate=src.b_gate.clone(),
                              act=src.act)

        def copy_pred(src):
            return B.SVDPredictor(src.q.clone(), src.l.clone(), src.tau.clone(), b=src.b.clone())
        n_layers = svd_layers
        layers = [layers[l] if l < svd_prepared else copy_layer(layers[l % svd_prepared]) for l in range(n_layers)]
        pred_seq = [pred_seq[l] if l < svd_prepared else copy_pred(pred_seq[l % svd_prepared]) for l in range(n_layers)]
        pred_par = [pred_par[l] if l < svd_prepared else copy_pred(pred_par[l % svd_prepared]) for l in range(n_layers)]
        torch.cuda.synchronize()
        ws = B.workspace(B.sparse_ffn_workspace_size(layers[0], 1))
        wsp_ = B.workspace(max(B.svd_predict_workspace_size(pred_seq[0]), B.svd_predict_workspace_size(pred_par[0])))
        X = xtok(w3, (n_warm + n_steps, n_layers, d), inputs.STREAM_DECODE)
        y = torch.zeros((n_layers, d), dtype=torch.float32, device=dev)
        cand = torch.zeros((n_layers, f), dtype=torch.int32, device=dev)
        ncand = torch.zeros((n_layers, 1), dtype=torch.int32, device=dev)
        nact = torch.zeros((n_layers, 1), dtype=torch.int32, device=dev)

        def predict(preds, tok, l):
            return (lib.svd_predict, (ctypes.byref(preds[l].c), X[tok, l].data_ptr(), cand[l].data_ptr(),
                                      ncand[l].data_ptr(), None, wsp_.data_ptr(), wsp_.numel()))

        def seq_calls(tok, l, counts=False):
            return [predict(pred_seq, tok, l),
                    (lib.sparse_ffn_decode, (ctypes.byref(layers[l].c), X[tok, l].data_ptr(), 1, None,
                                             cand[l].data_ptr(), ncand[l].data_ptr(), None, y[l].data_ptr(), None,
                                             nact[l].data_ptr() if counts else None, ws.data_ptr(), ws.numel()))]

        def par_calls(tok, l):
            return [predict(pred_par, tok, l),
                    (lib.sparse_ffn_decode_parallel, (ctypes.byref(layers[l].c), X[tok, l].data_ptr(), cand[l].data_ptr(),
                                                      ncand[l].data_ptr(), y[l].data_ptr(), ws.data_ptr(), ws.numel()))]

        def leg(calls):
            steps = [[c for l in range(n_layers) for c in calls(tok, l)] for tok in range(n_warm, n_warm + n_steps)]
            time_mixed(torch, [[c for l in range(n_layers) for c in calls(tok, l)] for tok in range(n_warm)], mode)
            return time_mixed(torch, steps, mode) * 1e3 / (n_steps * n_layers)

        # densities: untimed passes over the timed tokens
        dc, da, dcp = [], [], []
        for tok in range(n_warm, n_warm + n_steps):
            for l in range(n_layers):
                for fn, a in seq_calls(tok, l, True):
                    fn(*a, torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            dc.append(ncand.float().mean().item())
            da.append(nact.float().mean().item())
            for l in range(n_layers):
                fn, a = predict(pred_par, tok, l)
                fn(*a, torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            dcp.append(ncand.float().mean().item())
        nc, na, ncp = float(np.mean(dc)), float(np.mean(da)), float(np.mean(dcp))
        for name, r, calls, byts in (
                ("reglu_svd_r256_s50", 256, seq_calls, 2.0 * 256 * (d + f) + 8.0 * f + 2.0 * nc * d + 4.0 * na * d + 6.0 * d),
                ("reglu_svd_r1024_whitened_parallel", 1024, par_calls,
                 2.0 * 1024 * (d + f) + 8.0 * f + 6.0 * ncp * d + 6.0 * d)):
            us = leg(calls)
            preds = pred_seq if r == 256 else pred_par
            pred_us = time_mixed(torch, [[predict(preds, tok, l) for l in range(n_layers)]
                                         for tok in range(n_warm, n_warm + n_steps)], mode) * 1e3 / (n_steps * n_layers)
            out[name] = {"d": d, "f": f, "r": r, "s": w3.s, "layers_timed": n_layers,
                         "distinct_layer_values": svd_prepared, "us_per_layer": us,
                         "predictor_us": pred_us, "candidate_density": (nc if r == 256 else ncp) / f,
                         "algorithmic_bytes_per_layer": byts, "gbs": byts / (us * 1e-6) / 1e9,
                         "tokens_per_s": 1.0 / (n_layers * us * 1e-6)}
            if r == 256:
                out[name]["active_density"] = na / f
            log(f"  extra {name}: {us:.2f} us/layer (predictor {pred_us:.2f}), cand {out[name]['candidate_density']:.3f}")

        # the same two pipelines through the fused call: each tile predicts its own rows and
        # processes its candidates, no candidate list in between (same bytes)
        wsf = B.workspace(max(B.sparse_ffn_svd_workspace_size(layers[0], pred_seq[0]),
                              B.sparse_ffn_svd_workspace_size(layers[0], pred_par[0])))

        def fused(preds, pipe):
            return lambda tok, l: [(lib.sparse_ffn_decode_svd, (ctypes.byref(layers[l].c), ctypes.byref(preds[l].c),
                                                                X[tok, l].data_ptr(), pipe, y[l].data_ptr(), None, None,
                                                                wsf.data_ptr(), wsf.numel()))]
        for name, base, calls in (("reglu_svd_r256_s50_fused", "reglu_svd_r256_s50", fused(pred_seq, B.SFN_PIPE_SEQUENTIAL)),
                                  ("reglu_svd_r1024_whitened_parallel_fused", "reglu_svd_r1024_whitened_parallel",
                                   fused(pred_par, B.SFN_PIPE_PARALLEL))):
            us = leg(calls)
            byts = out[base]["algorithmic_bytes_per_layer"]
            out[name] = {"d": d, "f": f, "r": out[base]["r"], "s": w3.s, "layers_timed": n_layers,
                         "distinct_layer_values": svd_prepared, "us_per_layer": us,
                         "algorithmic_bytes_per_layer": byts, "gbs": byts / (us * 1e-6) / 1e9,
                         "tokens_per_s": 1.0 / (n_layers * us * 1e-6),
                         "speedup_over_unfused": out[base]["us_per_layer"] / us}
            log(f"  extra {name}: {us:.2f} us/layer ({out[name]['gbs']:.0f} GB/s), "
                f"{out[name]['speedup_over_unfused']:.2f}x the unfused calls")

        # the other two pairings of predictor and pipeline (SVDP Table 2 compares the
        # pipelines): rank 256 through the parallel pipeline, rank 1024 whitened through the
        # sequential one, whose active count comes from an untimed pass of the fused call
        nidx = torch.zeros((n_layers, 1), dtype=torch.int32, device=dev)
        dap = []
        for tok in range(n_warm, n_warm + n_steps):
            for l in range(n_layers):
                lib.sparse_ffn_decode_svd(ctypes.byref(layers[l].c), ctypes.byref(pred_par[l].c), X[tok, l].data_ptr(),
                                          B.SFN_PIPE_SEQUENTIAL, y[l].data_ptr(), cand[l].data_ptr(), nidx[l].data_ptr(),
                                          wsf.data_ptr(), wsf.numel(), torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            dap.append(nidx.float().mean().item())
        nap = float(np.mean(dap))
        for name, r, calls, byts in (
                ("reglu_svd_r256_parallel_fused", 256, fused(pred_seq, B.SFN_PIPE_PARALLEL),
                 2.0 * 256 * (d + f) + 8.0 * f + 6.0 * nc * d + 6.0 * d),
                ("reglu_svd_r1024_whitened_sequential_fused", 1024, fused(pred_par, B.SFN_PIPE_SEQUENTIAL),
                 2.0 * 1024 * (d + f) + 8.0 * f + 2.0 * ncp * d + 4.0 * nap * d + 6.0 * d)):
            us = leg(calls)
            out[name] = {"d": d, "f": f, "r": r, "s": w3.s, "layers_timed": n_layers,
                         "distinct_layer_values": svd_prepared, "us_per_layer": us,
                         "candidate_density": (nc if r == 256 else ncp) / f,
                         "algorithmic_bytes_per_layer": byts, "gbs": byts / (us * 1e-6) / 1e9,
                         "tokens_per_s": 1.0 / (n_layers * us * 1e-6)}
            if r == 1024:
                out[name]["active_density"] = nap / f
            log(f"  extra {name}: {us:.2f} us/layer ({out[name]['gbs']:.0f} GB/s)")

    if "tiny" in legs:
        # the tiny fp32 SwiGLU layer (d 256, f 688; 2.1 MB of weights, resident in the
        # caches): latency per call, all 64 decode tokens, threshold from 256 calibration
        # tokens; a graph of one call per token replayed back to back
        w0 = inputs.workload(0)
        l0 = [B.FFNLayer(*(torch.from_numpy(inputs.swiglu_layer(w0, 0)[k]).to(dev)
                           for k in ("w_gate", "w_up", "w_down_t")))]
        ws0 = B.workspace(B.sparse_ffn_workspace_size(l0[0], w0.n_cal))
        xc0 = torch.from_numpy(inputs.tokens(w0, w0.n_cal, inputs.STREAM_CAL)).to(dev)
        t0v = torch.zeros(1, dtype=torch.float32, device=dev)
        B.sparse_ffn_calibrate(l0[0], xc0, 0.5, t0v, ws0)
        X0 = torch.from_numpy(inputs.tokens(w0, w0.decode_tokens, inputs.STREAM_DECODE)).to(dev)
        y0 = torch.zeros((w0.decode_tokens, w0.d), dtype=torch.float32, device=dev)
        n0 = torch.zeros(w0.decode_tokens, dtype=torch.int32, device=dev)

        def tiny(tok, counts=False):
            return (lib.sparse_ffn_decode, (ctypes.byref(l0[0].c), X0[tok].data_ptr(), 1, t0v.data_ptr(), None, None,
                                            None, y0[tok].data_ptr(), None,
                                            n0[tok:tok + 1].data_ptr() if counts else None, ws0.data_ptr(),
                                            ws0.numel()))
        for tok in range(w0.decode_tokens):
            fn, a = tiny(tok, True)
            fn(*a, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        ntok = w0.decode_tokens
        # back to back: the 64 calls in one graph (per-call time in a stream of calls);
        # isolated: one graph per call, so each also pays the graph launch
        time_mixed(torch, [[tiny(tok) for tok in range(ntok)]], mode)
        ms = time_mixed(torch, [[tiny(tok) for tok in range(ntok)]], mode)
        ms_iso = time_mixed(torch, [[tiny(tok)] for tok in range(ntok)], mode)
        out["tiny_fp32_d256_f688_k50"] = {"d": w0.d, "f": w0.f, "dtype": "f32", "tokens": ntok,
                                          "us_per_call": ms * 1e3 / ntok,
                                          "us_per_call_isolated": ms_iso * 1e3 / ntok,
                                          "measured_density": float(n0.float().mean().item()) / w0.f,
                                          "note": "2.1 MB of weights stay in the caches: latency only"}
        log(f"  extra tiny fp32 layer: {ms * 1e3 / ntok:.2f} us per call back to back, "
            f"{ms_iso * 1e3 / ntok:.2f} us isolated")
        del l0, ws0, xc0, X0, y0

    # batch of 4 with per-token masks and the union gather (Llama-3-8B shape), and batch 1
    w2 = inputs.workload(2)
    if "b4" in legs:
        decode_leg("llama3_8b_b4_k50", w2, w2.d, w2.f, 4, 0.5, w2.layers)
        decode_leg("llama3_8b_b4_k60", w2, w2.d, w2.f, 4, 0.6, w2.layers)
    if "b1" in legs:
        decode_leg("llama3_8b_b1_k50", w2, w2.d, w2.f, 1, 0.5, w2.layers)
        decode_leg("llama3_8b_b1_k60", w2, w2.d, w2.f, 1, 0.6, w2.layers)
    # sparse decode at the Llama-3-70B shape (d 8192: two 16-byte chunks per thread)
    w4 = inputs.workload(4)
    if "70b" in legs:
        decode_leg("llama3_70b_b1_k50", w4, w4.d, w4.f, 1, 0.5, w4.layers)
    if "chunk" in legs:
        chunk_leg(w4)
    if "sirius" in legs:
        sirius_leg(w4)
    if "svd" in legs:
        svd_legs()
    return out



def cpu_baseline(stack, k, budget_s):
    """The oracle as it stands, timed on this host on a bounded sample: whole layers,
    weights widened to float64 beforehand (not timed), tokens one at a time."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    torch = stack.torch
    per = []
    layers_done = 0
    spent = 0.0
    t_host = stack.thr[k].cpu().numpy()
    for l in range(stack.L):
        if spent > budget_s and layers_done >= 1:
            break
        mats = [oracle.bf16_to_f64(m.view(torch.int16).cpu().numpy().view(np.uint16))
                for m in (stack.layers[l].w_gate, stack.layers[l].w_up, stack.layers[l].w_down_t)]
        for tok in range(3):
            x = oracle.bf16_to_f64(stack.X[tok, l].view(torch.int16).cpu().numpy().view(np.uint16))
            t0 = time.perf_counter()
            oracle.cats_decode(mats[0], mats[1], mats[2], x[None, :], float(t_host[l]))
            dt = time.perf_counter() - t0
            per.append(dt)
            spent += dt
        layers_done += 1
        del mats
    per_layer_token = float(np.median(per))
    tok_s = 1.0 / (per_layer_token * stack.L)
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": tok_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{layers_done} of {stack.L} layers x 3 tokens, median per-layer time x {stack.L} layers; "
                      f"float64 dense FFN then CATS mask (numpy), weights widened before timing",
            "cpu_model": cpu_model, "per_layer_token_ms": per_layer_token * 1e3}


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.command)
        return 0
    if args.summarize_traffic:
        return write_traffic(args.summarize_traffic, args.copy_probe << 20, args.command)
    if args.summarize_kernel_traffic:
        return summarize_kernel_traffic(*args.summarize_kernel_traffic, args.copy_probe << 20, args.command)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this library has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2
    import numpy as np
    import torch
    from contextual_activation_sparsity_amd import binding as B
    from contextual_activation_sparsity_amd import inputs

    if args.copy_probe:
        # a plain elementwise kernel of known traffic: reads n bytes, writes n bytes
        n = args.copy_probe << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"copy probe: 3 elementwise copies of {n} bytes")
        del src, dst
    K, W = args.steps, args.warmup
    sweep = [float(s) for s in args.sweep.split(",") if s.strip()] if args.sweep else []
    n_tok = K + W
    log(f"building stack: {args.layers} layers, {n_tok} tokens")
    stack = Stack(B, inputs, torch, args.layers, n_tok)
    d, f, L = stack.d, stack.f, stack.L
    lib = stack.lib
    for k in [args.sparsity] + sweep:
        stack.calibrate(k)
    log("calibrated thresholds for " + ", ".join(str(k) for k in [args.sparsity] + sweep))
    stream = torch.cuda.current_stream().cuda_stream

    def measure(k, steps_tok, mode):
        # densities: untimed pass with counts (identical masks: the kernel is deterministic)
        run_calls(lib.sparse_ffn_decode, [a for tok in steps_tok for a in stack.decode_args(tok, k, stream, True)])
        torch.cuda.synchronize()
        nact = stack.n_act[steps_tok].cpu().numpy().astype(np.float64)  # [steps, L]
        warm = [stack.decode_args(tok, k, stream) for tok in range(W)]
        timed = [stack.decode_args(tok, k, stream) for tok in steps_tok]
        time_steps(torch, lib.sparse_ffn_decode, warm, mode)
        ms = time_steps(torch, lib.sparse_ffn_decode, timed, mode)
        # algorithmic bytes: all gate rows, the active up and down rows, x in, y out
        bytes_tok = (L * (2.0 * f * d + 2.0 * d + 4.0 * d) + 4.0 * d * nact.sum(axis=1)).mean()
        return ms, nact, bytes_tok

    steps_tok = list(range(W, W + K))
    log(f"timing {K} steps at sparsity {args.sparsity} ({args.mode})")
    ms, nact, bytes_tok = measure(args.sparsity, steps_tok, args.mode)
    ms_step = ms / K
    tok_s = 1e3 / ms_step
    log(f"  {ms_step:.3f} ms/step, {tok_s:.1f} tokens/s, density {nact.mean() / f:.4f}")

    # roofline of one decode call: the timed region above, per call
    call_us = ms_step * 1e3 / L
    per_call_bytes = 2.0 * f * d + 6.0 * d + 4.0 * d * nact.mean()
    achieved = per_call_bytes / (call_us * 1e-6) / 1e9
    # the gate kernel alone: calls that request no output launch only the gate kernel
    gate_steps = [[a[:7] + (None, None, None) + a[10:] for a in stack.decode_args(tok, args.sparsity, stream)]
                  for tok in steps_tok]
    time_steps(torch, lib.sparse_ffn_decode, gate_steps[:W], args.mode)
    gate_us = time_steps(torch, lib.sparse_ffn_decode, gate_steps, args.mode) * 1e3 / (K * L)
    gate_bytes = 2.0 * f * d + 2.0 * d
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        if tr.get("kernel_hash") == kernel_hash():
            traffic = tr.get("bytes_per_call")
    if traffic is not None and abs(args.sparsity - 0.5) > 1e-9:
        traffic = None  # the counters were taken at k = 0.5
    roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                # the rate on the bytes the counters saw (rows plus the partials written and
                # read back), beside the algorithmic rate above
                "traffic_gbs": traffic / (call_us * 1e-6) / 1e9 if traffic else None,
                "traffic_frac": traffic / (call_us * 1e-6) / 1e9 / PEAK_HBM_GBS if traffic else None,
                "kernel": "sparse_ffn_decode call (decode_gate_local_kernel + decode_reduce_kernel), "
                          "bf16, batch 1, d 4096, f 11008",
                "algorithmic_bytes_per_launch": per_call_bytes, "avg_launch_us": call_us, "launches": K * L,
                "stages": {"gate_kernel": {"us": gate_us, "bytes": gate_bytes,
                                           "gbs": gate_bytes / (gate_us * 1e-6) / 1e9},
                           "updown_and_reduce": {"us": call_us - gate_us, "bytes": per_call_bytes - gate_bytes,
                                                         "gbs": (per_call_bytes - gate_bytes)
                                                         / ((call_us - gate_us) * 1e-6) / 1e9}}}
    log(f"  decode call: {call_us:.2f} us, {achieved:.1f} GB/s algorithmic ({achieved / PEAK_HBM_GBS:.3f}); "
        f"gate kernel alone {gate_us:.2f} us")

    result_sweep = []
    for k in sweep:
        ms_k, nact_k, bytes_k = measure(k, steps_tok, args.mode)
        st = ms_k / K
        result_sweep.append({"sparsity": k, "tokens_per_s": 1e3 / st, "ms_per_step": st,
                             "measured_density": float(nact_k.mean() / f), "bytes_per_token": bytes_k,
                             "step_gbs": bytes_k / (st * 1e-3) / 1e9})
        log(f"  sparsity {k}: {1e3 / st:.1f} tokens/s, density {nact_k.mean() / f:.4f}")

    dense = None
    if not args.no_dense:
        warm = [stack.dense_args(tok, stream) for tok in range(W)]
        timed = [stack.dense_args(tok, stream) for tok in steps_tok]
        time_steps(torch, lib.ffn_dense_chunk, warm, args.mode)
        ms_d = time_steps(torch, lib.ffn_dense_chunk, timed, args.mode) / K
        dense = {"call": "ffn_dense_chunk n=1", "tokens_per_s": 1e3 / ms_d, "ms_per_step": ms_d,
                 "step_gbs": L * 3.0 * 2 * f * d / (ms_d * 1e-3) / 1e9,
                 "speedup_of_sparse": tok_s / (1e3 / ms_d)}
        log(f"  dense path: {1e3 / ms_d:.1f} tokens/s, sparse speedup {dense['speedup_of_sparse']:.3f}")

    extra = None
    if not args.no_extras:
        log("timing the other workloads")
        legs = tuple(x.strip() for x in args.legs.split(",") if x.strip())
        unknown = set(legs) - set(EXTRA_LEGS)
        if unknown:
            raise SystemExit(f"unknown --legs entries: {sorted(unknown)}")
        extra = extras(B, inputs, torch, args.mode, legs=legs, svd_layers=args.svd_layers,
                       svd_prepared=min(args.svd_prepared, args.svd_layers), svd_prep_host=args.svd_prep_host)

    t4 = None
    if not args.no_table4:
        log("fixed-sparsity protocol (predictor excluded)")
        t4 = table4(B, inputs, torch, args.mode, shapes=tuple(T4_SHAPES[int(i)] for i in args.t4_shapes.split(",") if i),
                    sparsities=tuple(float(v) for v in args.t4_sparsities.split(",") if v))

    quality = None
    if not args.no_quality:
        log("predictor quality (ROC AUC and recall against rank and s)")
        quality = predictor_quality(B, inputs, torch)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(stack, args.sparsity, args.cpu_budget_s)
        log(f"  cpu oracle {cpu['value']:.3f} tokens/s on {cpu['cores']} threads")

    line = {
        "metric": "sparse-FFN decode tokens/s and achieved HBM GB/s vs peak at 50-90% sparsity",
        "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": stack.w.name, "layers": L, "d": d, "f": f, "batch": 1, "sparsity": args.sparsity,
                   "calibration_tokens": stack.w.n_cal, "measured_density": float(nact.mean() / f),
                   "mode": args.mode, "bytes_per_token": bytes_tok,
                   "step_gbs": bytes_tok / (ms_step * 1e-3) / 1e9},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "dense_path": dense,
        "sweep": result_sweep,
        "extras": extra,
        "table4": t4,
        "predictor_quality": quality,
    }
    print(json.dumps(line), flush=True)
    return 0


T4_SHAPES = ((1, 4096, 11008), (2, 4096, 14336), (5, 3584, 18944))  # (workload, d, f)


def table4(B, inputs, torch, mode, n_steps=16, n_warm=3, n_layers=4, shapes=T4_SHAPES,
           sparsities=(0.2, 0.5, 0.8, 0.95)):
    """The fixed-sparsity protocol of "SVD Contextual Sparsity Predictors for Fast LLM
    Inference", Table 4: the same sparsity on every layer and on every projection, the
    gate included, predictor excluded. Each token and layer gets its own uniformly drawn
    neuron subset of size round((1 - s) f), ascending, run through the one-pass
    candidate path (sparse_ffn_decode_parallel, SiLU); the dense FFN is ffn_dense_chunk
    with one token on the same layers. Reported per shape and sparsity: time per layer,
    algorithmic bytes and rate, and the FFN speedup over the dense call."""
    lib = B.raw()
    dev = "cuda"
    rows = []
    for wi, d, f in shapes:
        w = inputs.workload(wi)
        layers = [B.FFNLayer(*(inputs.torch_gaussian_bf16((f, d), w.w_std, inputs.seed(wi, l, tid), dev)
                               for tid in (inputs.T_GATE, inputs.T_UP, inputs.T_DOWN))) for l in range(n_layers)]
        ws = B.workspace(B.sparse_ffn_workspace_size(layers[0], 16))
        wsp, wsb = ws.data_ptr(), ws.numel()
        g = torch.Generator(device=dev)
        g.manual_seed(1_000_000 * wi + inputs.STREAM_DECODE)
        X = torch.randn((n_warm + n_steps, n_layers, d), generator=g, device=dev).to(torch.bfloat16)
        y = torch.zeros((n_layers, d), dtype=torch.float32, device=dev)

        def dense(tok, l):
            return (lib.ffn_dense_chunk, (ctypes.byref(layers[l].c), X[tok, l].data_ptr(), 1, y[l].data_ptr(),
                                          wsp, wsb))
        time_mixed(torch, [[dense(tok, l) for l in range(n_layers)] for tok in range(n_warm)], mode)
        dense_us = time_mixed(torch, [[dense(tok, l) for l in range(n_layers)]
                                      for tok in range(n_warm, n_warm + n_steps)], mode) * 1e3 / (n_steps * n_layers)
        for s in sparsities:
            n = int(round((1.0 - s) * f))
            gm = torch.Generator(device=dev)
            gm.manual_seed(1_000_000 * wi + inputs.STREAM_MASK + int(round(1000 * s)))
            cand = torch.stack([torch.sort(torch.randperm(f, generator=gm, device=dev)[:n])[0]
                                for _ in range((n_warm + n_steps) * n_layers)]).to(torch.int32)
            cand = cand.view(n_warm + n_steps, n_layers, n).contiguous()
            ncand = torch.full((1,), n, dtype=torch.int32, device=dev)

            def par(tok, l):
                return (lib.sparse_ffn_decode_parallel, (ctypes.byref(layers[l].c), X[tok, l].data_ptr(),
                                                         cand[tok, l].data_ptr(), ncand.data_ptr(), y[l].data_ptr(),
                                                         wsp, wsb))
            time_mixed(torch, [[par(tok, l) for l in range(n_layers)] for tok in range(n_warm)], mode)
            us = time_mixed(torch, [[par(tok, l) for l in range(n_layers)]
                                    for tok in range(n_warm, n_warm + n_steps)], mode) * 1e3 / (n_steps * n_layers)
            byts = 6.0 * n * d + 4.0 * n + 2.0 * d + 4.0 * d
            rows.append({"d": d, "f": f, "sparsity": s, "rows": n, "us_per_layer": us, "dense_us_per_layer": dense_us,
                         "ffn_speedup": dense_us / us, "bytes_ratio": (6.0 * f * d) / byts,
                         "algorithmic_bytes": byts, "gbs": byts / (us * 1e-6) / 1e9})
            log(f"  d {d} f {f} sparsity {s}: {us:.2f} us/layer ({rows[-1]['gbs']:.0f} GB/s), dense {dense_us:.2f}, "
                f"speedup {dense_us / us:.2f}")
            del cand
        del layers, ws, X, y
    return {"protocol": "fixed sparsity on every layer and projection (gate included), uniformly drawn neuron "
                        "subsets per token and layer, predictor excluded; one-pass candidate path vs dense FFN call",
            "layers_timed": n_layers, "steps": n_steps, "rows": rows}


def predictor_quality(B, inputs, torch, ranks=(16, 32, 64, 128, 256, 512, 1024), n_eval=256,
                      svals=(0.1, 0.3, 0.5, 0.7, 0.9)):
    """Predictor diagnostics on one ReGLU layer of the synthetic recipe ("SVD Contextual
    Sparsity Predictors for Fast LLM Inference", Figures 2, 4, 5 and 7): ROC AUC of the
    library's predictor outputs against the true activity (gate > 0, from the library's
    own mask-only decode) at each rank, with plain and whitened factors; and recall,
    false-negative rate and candidate density of the candidate sets at calibrated
    thresholds for several s, and at the zero threshold. Two token distributions:
    isotropic x ~ N(0, I) as everywhere else, and anisotropic x ~ N(0, R diag(e) R^T)
    with eigenvalues e log-spaced over two decades, where whitening can matter."""
    import numpy as np
    from contextual_activation_sparsity_amd import diagnostics as dg
    from contextual_activation_sparsity_amd import prepare
    dev = "cuda"
    w3 = inputs.workload(3)
    d, f = w3.d, w3.f
    gen = lambda sd: torch.Generator(device=dev).manual_seed(sd)  # noqa: E731
    A = torch.randn((f, w3.rank), generator=gen(inputs.seed(3, 0, inputs.T_A)), device=dev) / np.sqrt(w3.rank)
    Bm = torch.randn((w3.rank, d), generator=gen(inputs.seed(3, 0, inputs.T_B)), device=dev) * w3.w_std
    noise = torch.randn((f, d), generator=gen(inputs.seed(3, 0, inputs.T_NOISE)), device=dev) * w3.w_std
    wg = (A @ Bm + 0.1 * noise).to(torch.bfloat16)
    del A, Bm, noise
    bias = (-1.2815516 * wg.float().norm(dim=1)).contiguous()
    wu = inputs.torch_gaussian_bf16((f, d), w3.w_std, inputs.seed(3, 0, inputs.T_UP), dev)
    wd = inputs.torch_gaussian_bf16((f, d), w3.w_std, inputs.seed(3, 0, inputs.T_DOWN), dev)
    layer = B.FFNLayer(wg, wu, wd, b_gate=bias, act=B.SFN_ACT_RELU)
    ws = B.workspace(B.sparse_ffn_workspace_size(layer, 1))
    zero = torch.zeros(1, dtype=torch.float32, device=dev)
    n_cal = 2 * d
    z = torch.randn((n_cal + n_eval, d), generator=gen(1_000_000 * 3 + inputs.STREAM_TAU), device=dev)
    # random rotation, orthogonalized on the host
    Rm = torch.from_numpy(np.linalg.qr(np.random.default_rng(1_000_000 * 3 + 999_005).standard_normal((d, d)))[0])
    Rm = Rm.to(device=dev, dtype=torch.float32)
    e = torch.logspace(-1.0, 1.0, d, device=dev)
    e = e * (d / e.sum())  # mean eigenvalue 1, so the gate scale is unchanged on average
    out = {"layer": "reglu d 4096 f 11008, gate rank 256 + noise", "eval_tokens": n_eval,
           "calibration_tokens": n_cal, "ranks": list(ranks), "tokens": {}}
    for tname, X in (("isotropic", z), ("anisotropic", (z * e.sqrt()) @ Rm.T)):
        X = X.to(torch.bfloat16)
        xc, xe = X[:n_cal], X[n_cal:]
        # true activity of the evaluation tokens from the library: ReLU(g) > 0
        idx = torch.zeros((n_eval, f), dtype=torch.int32, device=dev)
        cnt = torch.zeros(n_eval, dtype=torch.int32, device=dev)
        for j in range(n_eval):
            B.sparse_ffn_decode(layer, xe[j:j + 1], zero, ws, y=None, active_idx=idx[j:j + 1], n_active=cnt[j:j + 1])
        act = dg.masks_from_lists(idx, cnt, f)
        gcal = xc.float() @ wg.float().t() + bias
        res = {"active_density": float(act.float().mean().item()), "auc": {}, "thresholds": []}
        for whiten in (False, True):
            facs = prepare.svd_factors_ranks(wg, ranks, x_cal=xc if whiten else None)
            aucs = {}
            for r, (q, lf) in facs.items():
                pred = B.SVDPredictor(q, lf, torch.zeros(f, dtype=torch.float32, device=dev), b=bias)
                wsp = B.workspace(B.svd_predict_workspace_size(pred))
                P = torch.zeros((n_eval, f), dtype=torch.float32, device=dev)
                cand = torch.zeros(f, dtype=torch.int32, device=dev)
                nc = torch.zeros(1, dtype=torch.int32, device=dev)
                for j in range(n_eval):
                    B.svd_predict(pred, xe[j:j + 1], cand, nc, wsp, p_out=P[j])
                aucs[r] = dg.roc_auc(P, act)
                if r in (256, 1024):
                    pcal = prepare.predictions(q, lf, xc.float(), bias)
                    for sv in (None,) + tuple(svals):
                        tau = (torch.zeros(f, dtype=torch.float32, device=dev) if sv is None
                               else prepare.calibrate_tau(pcal, gcal, sv))
                        pr = B.SVDPredictor(q, lf, tau, b=bias)
                        ci = torch.zeros((n_eval, f), dtype=torch.int32, device=dev)
                        cc = torch.zeros(n_eval, dtype=torch.int32, device=dev)
                        for j in range(n_eval):
                            B.svd_predict(pr, xe[j:j + 1], ci[j], cc[j:j + 1], wsp)
                        cm = dg.masks_from_lists(ci, cc, f)
                        rc = dg.recall(cm, act)
                        res["thresholds"].append({"r": r, "whitened": whiten, "s": sv if sv is not None else "zero",
                                                  "recall": rc, "false_negative_rate": 1.0 - rc,
                                                  "candidate_density": float(cm.float().mean().item())})
                    del pcal
            res["auc"]["whitened" if whiten else "plain"] = aucs
            log(f"  {tname} tokens, {'whitened' if whiten else 'plain'} factors: AUC "
                + " ".join(f"r{r} {a:.4f}" for r, a in aucs.items()))
        for t in res["thresholds"]:
            log(f"    r {t['r']} {'whitened' if t['whitened'] else 'plain'} s {t['s']}: recall {t['recall']:.4f}, "
                f"candidates {t['candidate_density']:.3f}")
        out["tokens"][tname] = res
    return out


def summarize_kernel_traffic(fetch_dir, write_dir, probe, command):
    """Markdown table of HBM bytes per dispatch of each of the library's kernels, from a
    FETCH_SIZE and a WRITE_SIZE --pmc run of the same command with the copy probe, each
    counter scaled so that the probe's copy of `probe` bytes reads (writes) exactly `probe`
    bytes. A kernel instance that serves several workloads (one grid, different row
    counts) reads different amounts per dispatch: its dispatches are split into clusters
    of bytes read (a new cluster wherever the sorted values jump by more than 5%), and each
    cluster gets a line with its median read and the median write of the same dispatches
    (the two runs dispatch in the same order, so the n-th dispatch of an instance is the
    same call in both)."""
    import statistics
    if probe <= 0:
        raise SystemExit("--copy-probe MIB must give the probe's size")
    vals, scale = {}, {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per, copies = {}, []
        rows = sorted((r for r in _csv_rows(d, "counter_collection.csv") if r.get("Counter_Name") == counter),
                      key=lambda r: int(r["Dispatch_Id"]))
        for r in rows:
            name = r["Kernel_Name"]
            v = float(r["Counter_Value"]) * 1024.0
            if _short(name) == COPY_KERNEL:
                copies.append(v)
                continue
            if "sfn::" not in name:
                continue
            wgs = int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"]))
            per.setdefault((_short(name, keep_args=True), wgs, int(r["Workgroup_Size"])), []).append(v)
        if not copies:
            raise SystemExit(f"{counter}: the copy probe's kernel is missing")
        scale[counter] = probe / statistics.median(copies)
        vals[counter] = {k: [x * scale[counter] for x in v] for k, v in per.items()}
    out = ["# rocprofv3 HBM traffic per dispatch", "", "Commands:", "", "```", command or "(not recorded)", "```", "",
           f"FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of each kernel, scaled by what the counters read for a "
           f"plain elementwise copy (torch.neg) of {probe >> 20} MiB in the same run: FETCH x "
           f"{scale['FETCH_SIZE']:.4f}, WRITE x {scale['WRITE_SIZE']:.4f}. One line per cluster of dispatches that "
           f"read about the same bytes (an instance serving several workloads has several).", "",
           "| kernel | workgroups x threads | dispatches | read MB (median) | read MB (min-max) | written MB (median) |",
           "|---|---|---|---|---|---|"]
    lines = []
    for key, fv in vals["FETCH_SIZE"].items():
        wv = vals["WRITE_SIZE"].get(key, [])
        paired = len(wv) == len(fv)
        order = sorted(range(len(fv)), key=lambda i: fv[i])
        clusters, cur = [], [order[0]]
        for a, b in zip(order, order[1:]):
            if fv[b] > 1.05 * fv[a] + 1e3:
                clusters.append(cur)
                cur = []
            cur.append(b)
        clusters.append(cur)
        for c in clusters:
            rd = [fv[i] for i in c]
            wr = statistics.median([wv[i] for i in c]) / 1e6 if paired else float("nan")
            lines.append((statistics.median(rd), f"| `{key[0]}` | {key[1]} x {key[2]} | {len(c)} | "
                                                 f"{statistics.median(rd) / 1e6:.2f} | {min(rd) / 1e6:.2f}-"
                                                 f"{max(rd) / 1e6:.2f} | {wr:.2f} |"))
    out += [ln for _, ln in sorted(lines, key=lambda t: -t[0])]
    print("\n".join(out))
    return 0


def write_traffic(dirs, probe, command):
    """HBM bytes per decode call: FETCH_SIZE and WRITE_SIZE of the kernels of a batch-1
    decode call, each counter scaled so that the probe's copy of `probe` bytes reads
    (writes) exactly `probe` bytes."""
    if probe <= 0:
        raise SystemExit("--copy-probe MIB must give the probe's size")
    res = summarize_traffic(dirs[0], dirs[1], probe)
    per_call = 0.0
    detail = {}
    for counter, r in res.items():
        scale = probe / r["copy_probe_bytes_counted"]
        ks = {k: v * scale for k, v in r["per_kernel_bytes"].items() if k in CALL_KERNELS}
        detail[counter] = {"scale": scale, "probe_counted_bytes": r["copy_probe_bytes_counted"],
                           "per_kernel_bytes": ks}
        per_call += sum(ks.values())
    out = {"kernel_hash": kernel_hash(), "bytes_per_call": per_call, "counters": detail, "command": command,
           "note": "FETCH_SIZE and WRITE_SIZE (KiB per dispatch, median over dispatches) of the kernels of "
                   "a batch-1 decode call, summed; each counter scaled by probe bytes / what it reads for a plain elementwise "
                   "copy (torch.neg) of 1 GiB in the same run. kernel_hash covers the decode kernel sources."}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
