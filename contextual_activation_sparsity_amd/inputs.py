"""Seeded synthetic inputs shared by the library's tests, the benchmark and the oracle tests.

This module holds data generation only -- shapes, distributions, seeds and the
float32 -> bfloat16 storage conversion -- and none of the sparse FFN's arithmetic. It
imports numpy (and torch, lazily, for the on-device generator the benchmark uses).

Workloads. The source pages measure on trained models and datasets that are not
available here, so every workload is synthetic at the pages' shapes
("SVD Contextual Sparsity Predictors for Fast LLM Inference", Table 12: hidden 4096 /
intermediate 11008 and 4096 / 14336; the Sirius summary's Llama-3-8B and -70B models):
Gaussian weights and tokens, with the recipes below.

Seeds. numpy ``Generator(PCG64(seed))`` with
``seed = 1_000_000 * workload + 1000 * layer + tensor_id`` (tensor ids: gate 0, up 1,
down 2, A 3, B 4, noise 5); calibration tokens use ``1_000_000 * workload + 999_001``,
decode tokens ``... + 999_002``, predictor-threshold calibration tokens
``... + 999_003``, fixed-density masks ``... + 999_004``.
"""

from dataclasses import dataclass, field
from typing import Tuple

import numpy as np

T_GATE, T_UP, T_DOWN, T_A, T_B, T_NOISE = 0, 1, 2, 3, 4, 5
STREAM_CAL, STREAM_DECODE, STREAM_TAU, STREAM_MASK = 999_001, 999_002, 999_003, 999_004

# z such that P(Z > z) = 0.1 for a standard normal Z (the 90% quantile).
_Z90 = 1.2815515655446004


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    d: int
    f: int
    layers: int
    dtype: str  # "f32" or "bf16": weights and tokens
    w_std: float  # standard deviation of the weight entries
    act: str = "silu"
    sparsities: Tuple[float, ...] = (0.5,)
    batches: Tuple[int, ...] = (1,)
    n_cal: int = 256
    decode_tokens: int = 64
    warmup_tokens: int = 8
    rank: int = 0  # SVD predictor rank (ReGLU workload)
    s: float = 0.0  # predictor-threshold hyperparameter (ReGLU workload)
    n_tau_cal: int = 0
    chunk: int = 0  # dense verification chunk (tokens)
    extra: dict = field(default_factory=dict)


WORKLOADS = (
    Workload(0, "tiny_swiglu_d256_f688_f32", 256, 688, 1, "f32", 1.0 / 16.0,
             sparsities=(0.5,)),
    Workload(1, "llama2_7b_ffn_d4096_f11008_bf16_l32", 4096, 11008, 32, "bf16", 0.02,
             sparsities=(0.5, 0.7, 0.8, 0.9)),
    Workload(2, "llama3_8b_ffn_d4096_f14336_bf16_l32", 4096, 14336, 32, "bf16", 0.02,
             sparsities=(0.5, 0.6), batches=(1, 4)),
    Workload(3, "reglu_svd_ffn_d4096_f11008_r256_bf16", 4096, 11008, 32, "bf16", 0.02,
             act="relu", rank=256, s=0.5, n_tau_cal=1024),
    Workload(4, "llama3_70b_ffn_d8192_f28672_bf16_l8", 8192, 28672, 8, "bf16", 0.02,
             sparsities=(0.5,), chunk=16),
    # SparseQwen2-7B FFN shape, for the fixed-sparsity protocol of SVDP Table 4 (random
    # neuron subsets at a fixed density on every layer, the gate included)
    Workload(5, "qwen2_7b_ffn_d3584_f18944_bf16", 3584, 18944, 28, "bf16", 0.02,
             sparsities=(0.2, 0.5, 0.8, 0.95)),
)


def workload(name_or_index):
    for w in WORKLOADS:
        if w.index == name_or_index or w.name == name_or_index:
            return w
    raise KeyError(name_or_index)


def seed(workload_index, layer, tensor_id):
    return 1_000_000 * int(workload_index) + 1000 * int(layer) + int(tensor_id)


def rng(s):
    return np.random.Generator(np.random.PCG64(s))


def f32_to_bf16_bits(a):
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the
    16-bit patterns as uint16. Inputs that are float64 are first rounded to float32."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(bits):
    """Widen bfloat16 patterns to float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _gaussian(s, shape, std):
    return rng(s).standard_normal(shape, dtype=np.float32) * np.float32(std)


def _store(a, dtype):
    return f32_to_bf16_bits(a) if dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32)


def swiglu_layer(w, layer, d=None, f=None):
    """Gate, up and transposed-down weights of one layer, each [f, d] row-major.

    Entries are iid N(0, w_std^2) in float32, stored as bfloat16 patterns (uint16) or
    float32 according to the workload. ``d``/``f`` override the workload's shape
    (smaller parity cases reuse a workload's recipe)."""
    d = w.d if d is None else d
    f = w.f if f is None else f
    out = {}
    for name, tid in (("w_gate", T_GATE), ("w_up", T_UP), ("w_down_t", T_DOWN)):
        out[name] = _store(_gaussian(seed(w.index, layer, tid), (f, d), w.w_std), w.dtype)
    return out


def reglu_layer(w, layer, d=None, f=None, rank_struct=256):
    """ReGLU layer with a low-rank-plus-noise gate and a per-neuron bias.

    W_gate = A B + 0.1 noise, A [f, 256] ~ N(0, 1/256), B [256, d] ~ N(0, 0.02^2),
    noise ~ N(0, 0.02^2), so gate entries have about the scale of the other weights.
    W_up and W_down^T ~ N(0, 0.02^2). The gate bias b_i = -z_0.9 ||w_i||_2 (w_i the
    stored bfloat16 row) makes neuron i active, g_i > 0, with probability 0.1 for
    x ~ N(0, I).
    """
    d = w.d if d is None else d
    f = w.f if f is None else f
    k = min(rank_struct, d, f)
    A = _gaussian(seed(w.index, layer, T_A), (f, k), 1.0 / np.sqrt(k))
    B = _gaussian(seed(w.index, layer, T_B), (k, d), w.w_std)
    noise = _gaussian(seed(w.index, layer, T_NOISE), (f, d), w.w_std)
    wg = A @ B + np.float32(0.1) * noise
    out = {
        "w_gate": f32_to_bf16_bits(wg),
        "w_up": f32_to_bf16_bits(_gaussian(seed(w.index, layer, T_UP), (f, d), w.w_std)),
        "w_down_t": f32_to_bf16_bits(_gaussian(seed(w.index, layer, T_DOWN), (f, d), w.w_std)),
    }
    rows = bf16_bits_to_f32(out["w_gate"]).astype(np.float64)
    out["b_gate"] = (-_Z90 * np.sqrt((rows * rows).sum(axis=1))).astype(np.float32)
    return out


def tokens(w, n, stream, d=None):
    """n tokens x ~ N(0, I_d), float32, rounded to bfloat16 for bfloat16 workloads
    (the library takes x in the weights' dtype). ``stream`` picks the seed family."""
    d = w.d if d is None else d
    x = rng(1_000_000 * w.index + stream).standard_normal((n, d), dtype=np.float32)
    return _store(x, w.dtype)


def random_masks(w, n, density, f=None, stream_offset=0):
    """n masks [n, f] (uint8) with exactly round(density f) active neurons each, drawn
    uniformly per token: the fixed-density protocol of "SVD Contextual Sparsity
    Predictors for Fast LLM Inference", Table 4 (same sparsity on every layer)."""
    f = w.f if f is None else f
    g = rng(1_000_000 * w.index + STREAM_MASK + stream_offset)
    n_act = int(round(density * f))
    m = np.zeros((n, f), dtype=np.uint8)
    for j in range(n):
        m[j, g.choice(f, size=n_act, replace=False)] = 1
    return m


def torch_gaussian_bf16(shape, std, s, device):
    """On-device N(0, std^2) weights rounded to bfloat16, seeded. Used by the
    benchmark to build multi-gigabyte stacks quickly; tests use the numpy recipes."""
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(s))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    return t.to(torch.bfloat16)
