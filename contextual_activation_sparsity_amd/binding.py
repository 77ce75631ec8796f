"""Thin ctypes binding of libsparse_ffn.so (declared in include/sparse_ffn.h).

The functions carry the C names and do argument marshalling only: they check that the
torch tensors they are given live on the GPU with the expected dtype and layout, pass
their device pointers and the current stream to the library, and raise on a negative
status. Every step of the computation runs in the library's HIP kernels; PyTorch only
owns the device memory and the stream. Importing this module fails loudly when the
library has not been built (``python -m contextual_activation_sparsity_amd.build``).
"""

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SFN_LIBRARY names another build of the same library (the host-sanitized one)
LIB_PATH = os.environ.get("SFN_LIBRARY") or os.path.join(_PKG, "libsparse_ffn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m contextual_activation_sparsity_amd.build` "
        "(hipcc, gfx950). There is no fallback implementation."
    )
_lib = ctypes.CDLL(LIB_PATH)

SFN_OK, SFN_EINVAL, SFN_ESHAPE, SFN_EDTYPE = 0, -1, -2, -3
SFN_EWORKSPACE, SFN_EALIGN, SFN_EUNSUPPORTED, SFN_EHIP, SFN_ETOOLARGE = -4, -5, -6, -7, -8
SFN_F32, SFN_BF16 = 0, 1
SFN_ACT_SILU, SFN_ACT_RELU = 0, 1
SFN_MAX_BATCH, SFN_MAX_CHUNK = 4, 16
SFN_PIPE_SEQUENTIAL, SFN_PIPE_PARALLEL = 0, 1
SFN_WORKSPACE_HEADER_BYTES, SFN_WORKSPACE_STATUS_OFFSET = 2048, 1024
SFN_STATUS_BALANCER_TIMEOUT, SFN_STATUS_PREDICTOR_TIMEOUT = 1, 2
SFN_NOALLOC_SCRATCH_BYTES = 32 << 20

EXPORTED = (
    "sparse_ffn_workspace_size",
    "svd_predict_workspace_size",
    "sparse_ffn_strerror",
    "sparse_ffn_calibrate",
    "sparse_ffn_decode",
    "sparse_ffn_decode_noalloc",
    "sparse_ffn_decode_parallel",
    "sparse_ffn_svd_workspace_size",
    "sparse_ffn_decode_svd",
    "svd_predict",
    "ffn_dense_chunk",
)


class sfn_ffn(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32), ("f", ctypes.c_int32), ("wdtype", ctypes.c_int32), ("act", ctypes.c_int32),
        ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down_t", ctypes.c_void_p),
        ("b_gate", ctypes.c_void_p),
    ]


class sfn_svd(ctypes.Structure):
    _fields_ = [
        ("d", ctypes.c_int32), ("f", ctypes.c_int32), ("r", ctypes.c_int32), ("reserved", ctypes.c_int32),
        ("q", ctypes.c_void_p), ("l", ctypes.c_void_p), ("b", ctypes.c_void_p), ("tau", ctypes.c_void_p),
    ]


_vp, _i32, _sz, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
_lib.sparse_ffn_workspace_size.argtypes = [ctypes.POINTER(sfn_ffn), _i32]
_lib.sparse_ffn_workspace_size.restype = _sz
_lib.svd_predict_workspace_size.argtypes = [ctypes.POINTER(sfn_svd)]
_lib.svd_predict_workspace_size.restype = _sz
_lib.sparse_ffn_strerror.argtypes = [ctypes.c_int]
_lib.sparse_ffn_strerror.restype = ctypes.c_char_p
_lib.sparse_ffn_calibrate.argtypes = [ctypes.POINTER(sfn_ffn), _vp, _i32, _f32, _vp, _vp, _vp, _sz, _vp]
_lib.sparse_ffn_calibrate.restype = ctypes.c_int
_lib.sparse_ffn_decode.argtypes = [ctypes.POINTER(sfn_ffn), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.sparse_ffn_decode.restype = ctypes.c_int
_lib.sparse_ffn_decode_noalloc.argtypes = [ctypes.POINTER(sfn_ffn), _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.sparse_ffn_decode_noalloc.restype = ctypes.c_int
_lib.sparse_ffn_decode_parallel.argtypes = [ctypes.POINTER(sfn_ffn), _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.sparse_ffn_decode_parallel.restype = ctypes.c_int
_lib.sparse_ffn_svd_workspace_size.argtypes = [ctypes.POINTER(sfn_ffn), ctypes.POINTER(sfn_svd)]
_lib.sparse_ffn_svd_workspace_size.restype = _sz
_lib.sparse_ffn_decode_svd.argtypes = [ctypes.POINTER(sfn_ffn), ctypes.POINTER(sfn_svd), _vp, _i32, _vp, _vp, _vp, _vp,
                                       _sz, _vp]
_lib.sparse_ffn_decode_svd.restype = ctypes.c_int
_lib.svd_predict.argtypes = [ctypes.POINTER(sfn_svd), _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.svd_predict.restype = ctypes.c_int
_lib.ffn_dense_chunk.argtypes = [ctypes.POINTER(sfn_ffn), _vp, _i32, _vp, _vp, _sz, _vp]
_lib.ffn_dense_chunk.restype = ctypes.c_int


class SparseFFNError(RuntimeError):
    def __init__(self, status, call):
        self.status = status
        super().__init__(f"{call}: status {status} ({sparse_ffn_strerror(status)})")


def _check(status, call):
    if status != SFN_OK:
        raise SparseFFNError(status, call)


def _ptr(t: Optional[torch.Tensor], name, dtype=None, numel=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor or None")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


_WDT = {torch.bfloat16: SFN_BF16, torch.float32: SFN_F32}


@dataclass
class FFNLayer:
    """One FFN layer's device tensors, each [f, d] row-major (w_down_t = W_down^T)."""

    w_gate: torch.Tensor
    w_up: Optional[torch.Tensor]
    w_down_t: Optional[torch.Tensor]
    b_gate: Optional[torch.Tensor] = None
    act: int = SFN_ACT_SILU

    def __post_init__(self):
        f, d = self.w_gate.shape
        dt = self.w_gate.dtype
        if dt not in _WDT:
            raise ValueError("weights must be bfloat16 or float32")
        for name in ("w_up", "w_down_t"):
            t = getattr(self, name)
            if t is not None and (tuple(t.shape) != (f, d) or t.dtype != dt):
                raise ValueError(f"{name} must be [{f}, {d}] {dt}")
        if self.b_gate is not None and (self.b_gate.dtype != torch.float32 or self.b_gate.numel() != f):
            raise ValueError("b_gate must be float32 [f]")
        self.d, self.f, self.dtype = d, f, dt
        self.c = sfn_ffn(
            d, f, _WDT[dt], int(self.act),
            _ptr(self.w_gate, "w_gate"), _ptr(self.w_up, "w_up"), _ptr(self.w_down_t, "w_down_t"),
            _ptr(self.b_gate, "b_gate", torch.float32),
        )


@dataclass
class SVDPredictor:
    """Rank-r predictor factors of one layer: q [r, d] bf16, l [f, r] bf16, b and tau [f] fp32."""

    q: torch.Tensor
    l: torch.Tensor
    tau: torch.Tensor
    b: Optional[torch.Tensor] = None

    def __post_init__(self):
        r, d = self.q.shape
        f, r2 = self.l.shape
        if r2 != r or self.q.dtype != torch.bfloat16 or self.l.dtype != torch.bfloat16:
            raise ValueError("q must be [r, d] and l [f, r], both bfloat16")
        self.d, self.f, self.r = d, f, r
        self.c = sfn_svd(d, f, r, 0, _ptr(self.q, "q"), _ptr(self.l, "l"),
                         _ptr(self.b, "b", torch.float32), _ptr(self.tau, "tau", torch.float32, f))


def sparse_ffn_workspace_size(layer: FFNLayer, max_tokens: int) -> int:
    return int(_lib.sparse_ffn_workspace_size(ctypes.byref(layer.c), int(max_tokens)))


def svd_predict_workspace_size(pred: SVDPredictor) -> int:
    return int(_lib.svd_predict_workspace_size(ctypes.byref(pred.c)))


def sparse_ffn_strerror(status: int) -> str:
    return _lib.sparse_ffn_strerror(int(status)).decode()


def workspace_status(ws: torch.Tensor) -> int:
    """The workspace status word (synchronises): 0, or the SFN_STATUS_* code of a bounded
    device-side wait that gave up during a call on this workspace."""
    off = SFN_WORKSPACE_STATUS_OFFSET
    return int(ws[off:off + 4].view(torch.int32).item())


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace of nbytes (its reserved first 2 KiB must start at zero)."""
    if nbytes <= 0:
        raise ValueError("workspace size query failed (invalid arguments)")
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def sparse_ffn_calibrate(layer: FFNLayer, x_cal: torch.Tensor, k: float, t_out: torch.Tensor,
                         ws: torch.Tensor, scores_out: Optional[torch.Tensor] = None, stream=None):
    n = x_cal.shape[0]
    st = _lib.sparse_ffn_calibrate(
        ctypes.byref(layer.c), _ptr(x_cal, "x_cal", layer.dtype, n * layer.d), int(n), float(k),
        _ptr(t_out, "t_out", torch.float32, 1),
        _ptr(scores_out, "scores_out", torch.float32, n * layer.f),
        _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sparse_ffn_calibrate")


def sparse_ffn_decode(layer: FFNLayer, x: torch.Tensor, t: Optional[torch.Tensor], ws: torch.Tensor,
                      y: Optional[torch.Tensor] = None, cand: Optional[torch.Tensor] = None,
                      n_cand: Optional[torch.Tensor] = None, mask_in: Optional[torch.Tensor] = None,
                      active_idx: Optional[torch.Tensor] = None, n_active: Optional[torch.Tensor] = None,
                      stream=None):
    B = x.shape[0] if x.dim() == 2 else 1
    st = _lib.sparse_ffn_decode(
        ctypes.byref(layer.c), _ptr(x, "x", layer.dtype, B * layer.d), int(B),
        _ptr(t, "t", torch.float32, 1), _ptr(cand, "cand", torch.int32), _ptr(n_cand, "n_cand", torch.int32, 1),
        _ptr(mask_in, "mask_in", torch.uint8, B * layer.f), _ptr(y, "y", torch.float32, B * layer.d),
        _ptr(active_idx, "active_idx", torch.int32, B * layer.f), _ptr(n_active, "n_active", torch.int32, B),
        _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sparse_ffn_decode")


def sparse_ffn_decode_noalloc(layer: FFNLayer, x: torch.Tensor, t: Optional[torch.Tensor],
                              y: Optional[torch.Tensor] = None, cand: Optional[torch.Tensor] = None,
                              n_cand: Optional[torch.Tensor] = None, mask_in: Optional[torch.Tensor] = None,
                              active_idx: Optional[torch.Tensor] = None, n_active: Optional[torch.Tensor] = None,
                              stream=None):
    B = x.shape[0] if x.dim() == 2 else 1
    st = _lib.sparse_ffn_decode_noalloc(
        ctypes.byref(layer.c), _ptr(x, "x", layer.dtype, B * layer.d), int(B),
        _ptr(t, "t", torch.float32, 1), _ptr(cand, "cand", torch.int32), _ptr(n_cand, "n_cand", torch.int32, 1),
        _ptr(mask_in, "mask_in", torch.uint8, B * layer.f), _ptr(y, "y", torch.float32, B * layer.d),
        _ptr(active_idx, "active_idx", torch.int32, B * layer.f), _ptr(n_active, "n_active", torch.int32, B),
        _stream(stream))
    _check(st, "sparse_ffn_decode_noalloc")


def sparse_ffn_decode_parallel(layer: FFNLayer, x: torch.Tensor, cand: torch.Tensor, n_cand: torch.Tensor,
                               ws: torch.Tensor, y: torch.Tensor, stream=None):
    st = _lib.sparse_ffn_decode_parallel(
        ctypes.byref(layer.c), _ptr(x, "x", layer.dtype, layer.d), _ptr(cand, "cand", torch.int32),
        _ptr(n_cand, "n_cand", torch.int32, 1), _ptr(y, "y", torch.float32, layer.d), _ptr(ws, "ws"),
        ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sparse_ffn_decode_parallel")


def sparse_ffn_svd_workspace_size(layer: FFNLayer, pred: SVDPredictor) -> int:
    return int(_lib.sparse_ffn_svd_workspace_size(ctypes.byref(layer.c), ctypes.byref(pred.c)))


def sparse_ffn_decode_svd(layer: FFNLayer, pred: SVDPredictor, x: torch.Tensor, ws: torch.Tensor,
                          y: Optional[torch.Tensor] = None, idx: Optional[torch.Tensor] = None,
                          n_idx: Optional[torch.Tensor] = None, pipeline: int = SFN_PIPE_SEQUENTIAL, stream=None):
    st = _lib.sparse_ffn_decode_svd(
        ctypes.byref(layer.c), ctypes.byref(pred.c), _ptr(x, "x", torch.bfloat16, layer.d), int(pipeline),
        _ptr(y, "y", torch.float32, layer.d), _ptr(idx, "idx", torch.int32, layer.f),
        _ptr(n_idx, "n_idx", torch.int32, 1), _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "sparse_ffn_decode_svd")


def svd_predict(pred: SVDPredictor, x: torch.Tensor, cand_idx: torch.Tensor, n_cand: torch.Tensor,
                ws: torch.Tensor, p_out: Optional[torch.Tensor] = None, stream=None):
    st = _lib.svd_predict(
        ctypes.byref(pred.c), _ptr(x, "x", torch.bfloat16, pred.d), _ptr(cand_idx, "cand_idx", torch.int32, pred.f),
        _ptr(n_cand, "n_cand", torch.int32, 1), _ptr(p_out, "p_out", torch.float32, pred.f),
        _ptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream))
    _check(st, "svd_predict")


def ffn_dense_chunk(layer: FFNLayer, x: torch.Tensor, y: torch.Tensor, ws: torch.Tensor, stream=None):
    n = x.shape[0]
    st = _lib.ffn_dense_chunk(
        ctypes.byref(layer.c), _ptr(x, "x", layer.dtype, n * layer.d), int(n),
        _ptr(y, "y", torch.float32, n * layer.d), _ptr(ws, "ws"), ws.numel() * ws.element_size(),
        _stream(stream))
    _check(st, "ffn_dense_chunk")


def raw():
    """The loaded ctypes library (for tests of the C-level error conventions)."""
    return _lib
