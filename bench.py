#!/usr/bin/env python3
"""Sparse-FFN decode benchmark on one MI355X.

Workload: the Llama-2-7B-shaped SwiGLU FFN stack -- 32 layers, hidden 4096,
intermediate 11008, bf16 weights ~ N(0, 0.02^2) generated on the device from fixed
seeds, batch 1, every layer of every token fed its own x ~ N(0, I) (bf16). CATS
thresholds are calibrated per layer by the library (256 calibration tokens) for the
headline sparsity (50%) and for the sweep points (70/80/90%).

A step is one decode token through all 32 layers (32 sparse_ffn_decode calls, one fused
kernel each). After W untimed warm-up steps, K steps are timed with HIP events on the
stream the kernels run on. The JSON line on stdout carries:
  value      decode tokens/s at the headline sparsity (inputs resident in HBM)
  roofline   the decode kernel's algorithmic bytes per launch (gate rows, the active
             up and down rows, x and y) over its average launch duration, measured with
             events around each launch, against the 8 TB/s HBM peak; `traffic` comes from
             the committed rocprofv3 counter summary when it matches the kernel source
  cpu_baseline  the CPU oracle (dense FFN then mask, numpy float64) timed on a bounded
             sample of layers and tokens of the same workload on this host
  dense_path the same stack through the library's dense path (ffn_dense_chunk, n = 1)
  sweep      tokens/s, density and GB/s at the other sparsities
Progress goes to stderr.
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
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
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
    return ap.parse_args()


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
        torch.cuda.synchronize()
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


def kernel_durations(torch, fn, step_args):
    """Per-launch durations (ms) from events recorded on the launch stream right before
    and after each call (one kernel per call)."""
    stream = torch.cuda.current_stream()
    evs = []
    torch.cuda.synchronize()
    for calls in step_args:
        for a in calls:
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            st = fn(*a)
            e.record(stream)
            if st != 0:
                raise RuntimeError(f"library call failed with status {st}")
            evs.append((s, e))
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in evs]


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
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2
    import numpy as np
    import torch
    from contextual_activation_sparsity_amd import binding as B
    from contextual_activation_sparsity_amd import inputs

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

    # roofline of the decode kernel: events around each launch of the timed tokens
    durs = kernel_durations(torch, lib.sparse_ffn_decode, [stack.decode_args(tok, args.sparsity, stream)
                                                            for tok in steps_tok])
    durs = np.array(durs)
    per_launch_bytes = 2.0 * f * d + 6.0 * d + 4.0 * d * nact.mean()
    avg_ms = float(durs.mean())
    achieved = per_launch_bytes / (avg_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        if tr.get("kernel_hash") == kernel_hash():
            traffic = tr.get("bytes_per_launch")
    roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                "kernel": "decode_kernel (bf16, batch 1, d 4096)",
                "algorithmic_bytes_per_launch": per_launch_bytes, "avg_launch_us": avg_ms * 1e3,
                "launches": int(durs.size)}
    log(f"  decode kernel: {avg_ms * 1e3:.2f} us/launch, {achieved:.1f} GB/s algorithmic ({achieved / PEAK_HBM_GBS:.3f})")

    result_sweep = []
    for k in sweep:
        ms_k, nact_k, bytes_k = measure(k, steps_tok, args.mode)
        st = ms_k / K
        result_sweep.append({"sparsity": k, "tokens_per_s": 1e3 / st, "ms_per_step": st,
                             "measured_density": float(nact_k.mean() / f),
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
                   "mode": args.mode, "step_gbs": bytes_tok / (ms_step * 1e-3) / 1e9},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "dense_path": dense,
        "sweep": result_sweep,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
