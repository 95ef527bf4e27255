"""Python binding of the MI355X Stable LatentMoE library (``libmoe_mi355x.so``).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their device pointers and the current HIP stream are passed to
the C ABI declared in ``include/moe_mi355x.h``, and every step of the layer
runs in the library's HIP kernels.  There is no fallback: if the library is
missing or fails to load, importing this package raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python sparse_moe_ffn_sigmoid_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

MOE_F32, MOE_BF16, MOE_MXFP4, MOE_MXFP4_A8, MOE_MXFP4_A4 = 0, 1, 2, 3, 4
MOE_QB_FROZEN, MOE_QB_BATCH = 0, 1
EXPORTED = ("moe_route_workspace_bytes", "moe_route_qb", "moe_route_sign",
            "moe_forward_workspace_bytes",
            "moe_latent_forward", "moe_status_str", "moe_stage_timing", "moe_stage_times",
            "moe_stage_name", "moe_mxfp8_quantize", "moe_mxfp4_quantize",
            "moe_route_qb_noalloc", "moe_backward_workspace_bytes", "moe_latent_backward",
            "moe_sgd_step", "moe_latent_backward_sgd", "moe_saved_activations_bytes",
            "moe_latent_forward_train", "moe_latent_backward_train")


class MoeShape(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("latent", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("routed_dtype", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("qb_mode", ctypes.c_int32),
                ("qb_max_rounds", ctypes.c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "w_router", "router_logit_offset", "w_down", "w_up", "w_gate", "w_uproj", "w_dn",
        "s_gate", "s_uproj", "s_dn", "rms_gamma", "ws_gate", "ws_up", "ws_down")]


_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
class MoeGrads(ctypes.Structure):
    _fields_ = [(f, ctypes.c_void_p) for f in (
        "dx", "d_w_router", "d_router_logit_offset", "d_w_down", "d_w_up", "d_w_gate",
        "d_w_uproj", "d_w_dn", "d_rms_gamma", "d_ws_gate", "d_ws_up", "d_ws_down")]


_lib.moe_route_workspace_bytes.argtypes = [_i32, _i32, _i32]
_lib.moe_route_workspace_bytes.restype = _sz
_lib.moe_route_qb.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                              _sz, _vp]
_lib.moe_route_qb.restype = ctypes.c_int
_lib.moe_route_sign.argtypes = [_vp, _i32, _i32, _i32, ctypes.c_double, _i32, _vp, _vp, _vp, _vp,
                                _vp, _vp, _sz, _vp]
_lib.moe_route_sign.restype = ctypes.c_int
_lib.moe_forward_workspace_bytes.argtypes = [ctypes.POINTER(MoeShape)]
_lib.moe_forward_workspace_bytes.restype = _sz
_lib.moe_latent_forward.argtypes = [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights), _vp,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moe_latent_forward.restype = ctypes.c_int
_lib.moe_status_str.argtypes = [ctypes.c_int]
_lib.moe_status_str.restype = ctypes.c_char_p
_lib.moe_stage_timing.argtypes = [ctypes.c_int]
_lib.moe_stage_timing.restype = ctypes.c_int
_lib.moe_stage_times.argtypes = [_vp, _vp, _i32]
_lib.moe_stage_times.restype = ctypes.c_int
_lib.moe_stage_name.argtypes = [ctypes.c_int]
_lib.moe_stage_name.restype = ctypes.c_char_p
_lib.moe_route_qb_noalloc.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                                      _vp]
_lib.moe_route_qb_noalloc.restype = ctypes.c_int
_lib.moe_backward_workspace_bytes.argtypes = [ctypes.POINTER(MoeShape)]
_lib.moe_backward_workspace_bytes.restype = _sz
_lib.moe_latent_backward.argtypes = [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights), _vp, _vp,
                                     _vp, _vp, _vp, ctypes.POINTER(MoeGrads), _vp, _sz, _vp]
_lib.moe_latent_backward.restype = ctypes.c_int
_lib.moe_sgd_step.argtypes = [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights),
                              ctypes.POINTER(MoeGrads), ctypes.c_float, _vp]
_lib.moe_sgd_step.restype = ctypes.c_int
_lib.moe_latent_backward_sgd.argtypes = [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights), _vp,
                                         _vp, _vp, _vp, _vp, ctypes.POINTER(MoeGrads),
                                         ctypes.c_float, _vp, _sz, _vp]
_lib.moe_latent_backward_sgd.restype = ctypes.c_int
_lib.moe_saved_activations_bytes.argtypes = [ctypes.POINTER(MoeShape)]
_lib.moe_saved_activations_bytes.restype = _sz
_lib.moe_latent_forward_train.argtypes = [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights),
                                          _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                          _vp, _sz, _vp]
_lib.moe_latent_forward_train.restype = ctypes.c_int
_lib.moe_latent_backward_train.argtypes = [ctypes.POINTER(MoeShape), ctypes.POINTER(MoeWeights),
                                           _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                           ctypes.POINTER(MoeGrads), ctypes.c_int, ctypes.c_float,
                                           _vp, _sz, _vp]
_lib.moe_latent_backward_train.restype = ctypes.c_int
_lib.moe_mxfp4_quantize.argtypes = [_vp, ctypes.c_int64, ctypes.c_int64, _vp, _vp, _vp]
_lib.moe_mxfp4_quantize.restype = ctypes.c_int
_lib.moe_mxfp8_quantize.argtypes = [_vp, ctypes.c_int64, ctypes.c_int64, _vp, _vp, _vp]
_lib.moe_mxfp8_quantize.restype = ctypes.c_int


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {_lib.moe_status_str(status).decode()} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    return _lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(t, name, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def route_workspace_bytes(T: int, n: int, k: int) -> int:
    return int(_lib.moe_route_workspace_bytes(T, n, k))


def route_qb(scores: torch.Tensor, k: int, bias: torch.Tensor | None = None,
             mode: int = MOE_QB_BATCH, max_rounds: int = 64, workspace=None):
    """Route fp32 scores [T, n] (device) to k experts per token.

    Returns dict(idx [T,k] int32, w [T,k] fp32, loads [n] int32, bias [n] fp64,
    info [4] int32) -- info = (quantile rounds, status, max |load-target|,
    augmenting-path moves).  ``bias`` (fp64 [n]) is the start / frozen bias.
    """
    dev = scores.device
    T, n = scores.shape
    _check(scores, "scores", torch.float32, (T, n), dev)
    b = torch.zeros(n, dtype=torch.float64, device=dev) if bias is None else bias.clone()
    _check(b, "bias", torch.float64, (n,), dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    loads = torch.empty(n, dtype=torch.int32, device=dev)
    info = torch.zeros(4, dtype=torch.int32, device=dev)
    need = route_workspace_bytes(T, n, k)
    ws = workspace if workspace is not None else torch.empty(max(need, 256), dtype=torch.uint8,
                                                             device=dev)
    st = _lib.moe_route_qb(_ptr(scores), T, n, k, mode, max_rounds, _ptr(b), _ptr(idx), _ptr(w),
                           _ptr(loads), _ptr(info), _ptr(ws), ws.numel(), _stream())
    if st != 0:
        raise MoeError(st, "moe_route_qb")
    return dict(idx=idx, w=w, loads=loads, bias=b, info=info)


def route_qb_noalloc(scores: torch.Tensor, k: int, bias: torch.Tensor | None = None,
                     mode: int = MOE_QB_BATCH, max_rounds: int = 64):
    """:func:`route_qb` through moe_route_qb_noalloc: the library's own
    per-device scratch array instead of a workspace (outputs are still
    allocated here, by torch)."""
    dev = scores.device
    T, n = scores.shape
    _check(scores, "scores", torch.float32, (T, n), dev)
    b = torch.zeros(n, dtype=torch.float64, device=dev) if bias is None else bias.clone()
    _check(b, "bias", torch.float64, (n,), dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    loads = torch.empty(n, dtype=torch.int32, device=dev)
    info = torch.zeros(4, dtype=torch.int32, device=dev)
    st = _lib.moe_route_qb_noalloc(_ptr(scores), T, n, k, mode, max_rounds, _ptr(b), _ptr(idx),
                                   _ptr(w), _ptr(loads), _ptr(info), _stream())
    if st != 0:
        raise MoeError(st, "moe_route_qb_noalloc")
    return dict(idx=idx, w=w, loads=loads, bias=b, info=info)


def route_sign(scores: torch.Tensor, k: int, step: float, max_rounds: int,
               bias: torch.Tensor | None = None, workspace=None):
    """DeepSeek-V3's fixed-step sign update of the bias on fp32 scores [T, n]
    (device), the baseline for Quantile Balancing.  Returns the dict of
    :func:`route_qb` with info = (updates, status, max |load-target|, 0)."""
    dev = scores.device
    T, n = scores.shape
    _check(scores, "scores", torch.float32, (T, n), dev)
    b = torch.zeros(n, dtype=torch.float64, device=dev) if bias is None else bias.clone()
    _check(b, "bias", torch.float64, (n,), dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    loads = torch.empty(n, dtype=torch.int32, device=dev)
    info = torch.zeros(4, dtype=torch.int32, device=dev)
    need = route_workspace_bytes(T, n, k)
    ws = workspace if workspace is not None else torch.empty(max(need, 256), dtype=torch.uint8,
                                                             device=dev)
    st = _lib.moe_route_sign(_ptr(scores), T, n, k, float(step), max_rounds, _ptr(b), _ptr(idx),
                             _ptr(w), _ptr(loads), _ptr(info), _ptr(ws), ws.numel(), _stream())
    if st != 0:
        raise MoeError(st, "moe_route_sign")
    return dict(idx=idx, w=w, loads=loads, bias=b, info=info)


def mxfp8_quantize(x: torch.Tensor):
    """bf16 rows [rows, K] (device, K a multiple of 32) -> (E4M3 codes uint8
    [rows, K], E8M0 scales uint8 [rows, K/32]), one scale per 32 elements."""
    rows, K = x.shape
    _check(x, "x", torch.bfloat16, (rows, K), x.device)
    codes = torch.empty((rows, K), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    st = _lib.moe_mxfp8_quantize(_ptr(x), rows, K, _ptr(codes), _ptr(scales), _stream())
    if st != 0:
        raise MoeError(st, "moe_mxfp8_quantize")
    return codes, scales


def mxfp4_quantize(x: torch.Tensor):
    """bf16 rows [rows, K] (device, K a multiple of 32) -> (E2M1 codes uint8
    [rows, K/2], two per byte, element 2i in the low nibble; E8M0 scales uint8
    [rows, K/32])."""
    rows, K = x.shape
    _check(x, "x", torch.bfloat16, (rows, K), x.device)
    codes = torch.empty((rows, K // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device=x.device)
    st = _lib.moe_mxfp4_quantize(_ptr(x), rows, K, _ptr(codes), _ptr(scales), _stream())
    if st != 0:
        raise MoeError(st, "moe_mxfp4_quantize")
    return codes, scales


GRAD_SHAPES = {  # gradient name -> (weight key, shape from (T, d, L, n, k, m, ms))
    "d_w_router": ("w_router", lambda T, d, L, n, k, m, ms: (n, d)),
    "d_router_logit_offset": ("router_logit_offset", lambda T, d, L, n, k, m, ms: (n,)),
    "d_w_down": ("w_down", lambda T, d, L, n, k, m, ms: (L, d)),
    "d_w_up": ("w_up", lambda T, d, L, n, k, m, ms: (d, L)),
    "d_w_gate": ("w_gate", lambda T, d, L, n, k, m, ms: (n, m, L)),
    "d_w_uproj": ("w_uproj", lambda T, d, L, n, k, m, ms: (n, m, L)),
    "d_w_dn": ("w_dn", lambda T, d, L, n, k, m, ms: (n, L, m)),
    "d_rms_gamma": ("rms_gamma", lambda T, d, L, n, k, m, ms: (L,)),
    "d_ws_gate": ("ws_gate", lambda T, d, L, n, k, m, ms: (ms, d)),
    "d_ws_up": ("ws_up", lambda T, d, L, n, k, m, ms: (ms, d)),
    "d_ws_down": ("ws_down", lambda T, d, L, n, k, m, ms: (d, ms)),
}


def latent_backward(shape: MoeShape, weights: dict, x: torch.Tensor, scores: torch.Tensor,
                    idx: torch.Tensor, w: torch.Tensor, dout: torch.Tensor, workspace=None):
    """Gradients of sum(out * dout) for a forward call with routing (scores
    [T,n] f32, idx [T,k] i32, w [T,k] f32), the selection held fixed.  Returns
    dict(dx, d_w_router, ...): fp32 weight gradients, dx in the activation
    dtype (bf16 layers only)."""
    dev = x.device
    T, d, l, n, k = shape.T, shape.d, shape.latent, shape.n_experts, shape.top_k
    m, ms = shape.inter, shape.shared_inter
    _check(x, "x", torch.bfloat16, (T, d), dev)
    _check(dout, "dout", torch.bfloat16, (T, d), dev)
    _check(scores, "scores", torch.float32, (T, n), dev)
    _check(idx, "idx", torch.int32, (T, k), dev)
    _check(w, "w", torch.float32, (T, k), dev)
    wts = MoeWeights(*[None if weights.get(f) is None else weights[f].data_ptr()
                       for f, _ in MoeWeights._fields_])
    out = {"dx": torch.empty((T, d), dtype=torch.bfloat16, device=dev)}
    for name, (key, fn) in GRAD_SHAPES.items():
        if weights.get(key) is None:
            out[name] = None
        else:
            out[name] = torch.empty(fn(T, d, l, n, k, m, ms), dtype=torch.float32, device=dev)
    grads = MoeGrads(*[None if out[f] is None else out[f].data_ptr() for f, _ in MoeGrads._fields_])
    need = _lib.moe_backward_workspace_bytes(ctypes.byref(shape))
    if need == 0:
        raise MoeError(-2, "moe_backward_workspace_bytes")
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=dev)
    st = _lib.moe_latent_backward(ctypes.byref(shape), ctypes.byref(wts), _ptr(x), _ptr(scores),
                                  _ptr(idx), _ptr(w), _ptr(dout), ctypes.byref(grads), _ptr(ws),
                                  ws.numel(), _stream())
    if st != 0:
        raise MoeError(st, "moe_latent_backward")
    return out


EXPERT_GRADS = ("d_w_gate", "d_w_uproj", "d_w_dn")


def latent_backward_sgd(shape: MoeShape, weights: dict, x: torch.Tensor, scores: torch.Tensor,
                        idx: torch.Tensor, w: torch.Tensor, dout: torch.Tensor, lr: float,
                        workspace=None):
    """latent_backward followed by sgd_step in one call, the routed experts'
    weight gradients applied in place without being stored.  Updates every
    weight tensor of `weights`; returns the other gradients (dx, d_w_router,
    ...; the three expert entries are None)."""
    dev = x.device
    T, d, l, n, k = shape.T, shape.d, shape.latent, shape.n_experts, shape.top_k
    m, ms = shape.inter, shape.shared_inter
    _check(x, "x", torch.bfloat16, (T, d), dev)
    _check(dout, "dout", torch.bfloat16, (T, d), dev)
    _check(scores, "scores", torch.float32, (T, n), dev)
    _check(idx, "idx", torch.int32, (T, k), dev)
    _check(w, "w", torch.float32, (T, k), dev)
    wts = MoeWeights(*[None if weights.get(f) is None else weights[f].data_ptr()
                       for f, _ in MoeWeights._fields_])
    out = {"dx": torch.empty((T, d), dtype=torch.bfloat16, device=dev)}
    for name, (key, fn) in GRAD_SHAPES.items():
        if weights.get(key) is None or name in EXPERT_GRADS:
            out[name] = None
        else:
            out[name] = torch.empty(fn(T, d, l, n, k, m, ms), dtype=torch.float32, device=dev)
    grads = MoeGrads(*[None if out[f] is None else out[f].data_ptr() for f, _ in MoeGrads._fields_])
    need = _lib.moe_backward_workspace_bytes(ctypes.byref(shape))
    if need == 0:
        raise MoeError(-2, "moe_backward_workspace_bytes")
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=dev)
    st = _lib.moe_latent_backward_sgd(ctypes.byref(shape), ctypes.byref(wts), _ptr(x),
                                      _ptr(scores), _ptr(idx), _ptr(w), _ptr(dout),
                                      ctypes.byref(grads), ctypes.c_float(lr), _ptr(ws),
                                      ws.numel(), _stream())
    if st != 0:
        raise MoeError(st, "moe_latent_backward_sgd")
    return out


def latent_backward_train(shape: MoeShape, weights: dict, x: torch.Tensor, scores: torch.Tensor,
                          idx: torch.Tensor, w: torch.Tensor, dout: torch.Tensor,
                          saved: torch.Tensor, lr=None, workspace=None):
    """The backward of a training forward (latent_forward with `saved`),
    reading the activations it kept.  lr None: every gradient, as
    latent_backward; else the SGD step is applied as in latent_backward_sgd
    (the experts' gradients in place, not returned)."""
    dev = x.device
    T, d, l, n, k = shape.T, shape.d, shape.latent, shape.n_experts, shape.top_k
    m, ms = shape.inter, shape.shared_inter
    _check(x, "x", torch.bfloat16, (T, d), dev)
    _check(dout, "dout", torch.bfloat16, (T, d), dev)
    _check(scores, "scores", torch.float32, (T, n), dev)
    _check(idx, "idx", torch.int32, (T, k), dev)
    _check(w, "w", torch.float32, (T, k), dev)
    _check(saved, "saved", torch.uint8, (saved.numel(),), dev)
    wts = MoeWeights(*[None if weights.get(f) is None else weights[f].data_ptr()
                       for f, _ in MoeWeights._fields_])
    out = {"dx": torch.empty((T, d), dtype=torch.bfloat16, device=dev)}
    for name, (key, fn) in GRAD_SHAPES.items():
        if weights.get(key) is None or (lr is not None and name in EXPERT_GRADS):
            out[name] = None
        else:
            out[name] = torch.empty(fn(T, d, l, n, k, m, ms), dtype=torch.float32, device=dev)
    grads = MoeGrads(*[None if out[f] is None else out[f].data_ptr() for f, _ in MoeGrads._fields_])
    need = _lib.moe_backward_workspace_bytes(ctypes.byref(shape))
    if need == 0:
        raise MoeError(-2, "moe_backward_workspace_bytes")
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=dev)
    st = _lib.moe_latent_backward_train(ctypes.byref(shape), ctypes.byref(wts), _ptr(x),
                                        _ptr(scores), _ptr(idx), _ptr(w), _ptr(dout),
                                        _ptr(saved), saved.numel(), ctypes.byref(grads),
                                        0 if lr is None else 1,
                                        ctypes.c_float(0.0 if lr is None else lr), _ptr(ws),
                                        ws.numel(), _stream())
    if st != 0:
        raise MoeError(st, "moe_latent_backward_train")
    return out


def sgd_step(shape: MoeShape, weights: dict, grads: dict, lr: float):
    """One gradient-descent step in place on the weight tensors of `weights`
    (w <- w - lr * g, fp32 operations, stored in each weight's type) from
    `grads` as returned by latent_backward (dx is not used)."""
    wts = MoeWeights(*[None if weights.get(f) is None else weights[f].data_ptr()
                       for f, _ in MoeWeights._fields_])
    gr = MoeGrads(*[None if f == "dx" or grads.get(f) is None else grads[f].data_ptr()
                    for f, _ in MoeGrads._fields_])
    for name, (key, _) in GRAD_SHAPES.items():
        wt, g = weights.get(key), grads.get(name)
        if (wt is None) != (g is None) or (g is not None and (
                g.dtype != torch.float32 or g.shape != wt.shape or not g.is_contiguous()
                or not wt.is_contiguous() or g.device != wt.device)):
            raise ValueError(f"sgd_step: {name} does not match {key}")
    st = _lib.moe_sgd_step(ctypes.byref(shape), ctypes.byref(wts), ctypes.byref(gr),
                           ctypes.c_float(lr), _stream())
    if st != 0:
        raise MoeError(st, "moe_sgd_step")


def make_shape(T, d, latent, n, k, inter, shared_inter, act_dtype, routed_dtype,
               rms_eps=1e-6, qb_mode=MOE_QB_BATCH, qb_max_rounds=64) -> MoeShape:
    return MoeShape(T, d, latent, n, k, inter, shared_inter, act_dtype, routed_dtype, rms_eps,
                    qb_mode, qb_max_rounds)


def forward_workspace_bytes(shape: MoeShape) -> int:
    return int(_lib.moe_forward_workspace_bytes(ctypes.byref(shape)))


_DT = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}


def saved_activations_bytes(shape: MoeShape) -> int:
    return int(_lib.moe_saved_activations_bytes(ctypes.byref(shape)))


def latent_forward(shape: MoeShape, weights: dict, x: torch.Tensor, bias=None,
                   scores_in=None, want_scores=False, workspace=None, saved=None):
    """One forward pass of the layer.

    ``saved``: a device uint8 buffer of saved_activations_bytes(shape) bytes;
    when given, the training forward also keeps there what
    latent_backward_train needs (bf16 layers).

    ``weights`` holds device tensors keyed as in ``moe_weights_t`` (MXFP4
    routed weights as uint8 codes plus ``s_gate``/``s_uproj``/``s_dn``).
    Returns dict(out, idx, w, loads, bias, info[, scores]).
    """
    dev = x.device
    T, d, l, n, k = shape.T, shape.d, shape.latent, shape.n_experts, shape.top_k
    m, ms = shape.inter, shape.shared_inter
    adt = _DT[shape.act_dtype]
    _check(x, "x", adt, (T, d), dev)
    _check(weights["w_router"], "w_router", torch.float32, (n, d), dev)
    if weights.get("router_logit_offset") is not None:
        _check(weights["router_logit_offset"], "router_logit_offset", torch.float32, (n,), dev)
    _check(weights["w_down"], "w_down", adt, (l, d), dev)
    _check(weights["w_up"], "w_up", adt, (d, l), dev)
    if shape.routed_dtype in (MOE_MXFP4, MOE_MXFP4_A8, MOE_MXFP4_A4):
        for nm, sn, rows, K in (("w_gate", "s_gate", m, l), ("w_uproj", "s_uproj", m, l),
                                ("w_dn", "s_dn", l, m)):
            _check(weights[nm], nm, torch.uint8, (n, rows, K // 2), dev)
            _check(weights[sn], sn, torch.uint8, (n, rows, K // 32), dev)
    else:
        rdt = _DT[shape.routed_dtype]
        _check(weights["w_gate"], "w_gate", rdt, (n, m, l), dev)
        _check(weights["w_uproj"], "w_uproj", rdt, (n, m, l), dev)
        _check(weights["w_dn"], "w_dn", rdt, (n, l, m), dev)
    _check(weights["rms_gamma"], "rms_gamma", torch.float32, (l,), dev)
    _check(weights["ws_gate"], "ws_gate", adt, (ms, d), dev)
    _check(weights["ws_up"], "ws_up", adt, (ms, d), dev)
    _check(weights["ws_down"], "ws_down", adt, (d, ms), dev)
    if scores_in is not None:
        _check(scores_in, "scores_in", torch.float32, (T, n), dev)
    wts = MoeWeights(*[None if weights.get(f) is None else weights[f].data_ptr()
                       for f, _ in MoeWeights._fields_])
    out = torch.empty((T, d), dtype=adt, device=dev)
    b = torch.zeros(n, dtype=torch.float64, device=dev) if bias is None else bias.clone()
    _check(b, "bias", torch.float64, (n,), dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    loads = torch.empty(n, dtype=torch.int32, device=dev)
    info = torch.zeros(4, dtype=torch.int32, device=dev)
    scores = torch.empty((T, n), dtype=torch.float32, device=dev) if want_scores else None
    need = forward_workspace_bytes(shape)
    if need == 0:
        raise MoeError(-1, "moe_forward_workspace_bytes")
    ws = workspace if workspace is not None else torch.empty(need, dtype=torch.uint8, device=dev)
    if saved is not None:
        _check(saved, "saved", torch.uint8, (saved.numel(),), dev)
        st = _lib.moe_latent_forward_train(ctypes.byref(shape), ctypes.byref(wts), _ptr(x),
                                           _ptr(out), _ptr(b), _ptr(scores_in), _ptr(scores),
                                           _ptr(idx), _ptr(w), _ptr(loads), _ptr(info),
                                           _ptr(saved), saved.numel(), _ptr(ws), ws.numel(),
                                           _stream())
        if st != 0:
            raise MoeError(st, "moe_latent_forward_train")
    else:
        st = _lib.moe_latent_forward(ctypes.byref(shape), ctypes.byref(wts), _ptr(x), _ptr(out),
                                     _ptr(b), _ptr(scores_in), _ptr(scores), _ptr(idx), _ptr(w),
                                     _ptr(loads), _ptr(info), _ptr(ws), ws.numel(), _stream())
        if st != 0:
            raise MoeError(st, "moe_latent_forward")
    res = dict(out=out, idx=idx, w=w, loads=loads, bias=b, info=info)
    if want_scores:
        res["scores"] = scores
    return res


def stage_timing(enable: bool) -> None:
    """Start (and reset) or stop per-stage HIP-event timing in the library."""
    _lib.moe_stage_timing(1 if enable else 0)


def stage_times() -> dict:
    """{stage name: (total ms, launches)} since the last stage_timing(True);
    synchronise the streams first."""
    tot = (ctypes.c_double * 16)()
    cnt = (ctypes.c_int32 * 16)()
    n = _lib.moe_stage_times(ctypes.cast(tot, ctypes.c_void_p), ctypes.cast(cnt, ctypes.c_void_p), 16)
    if n < 0:
        raise MoeError(n, "moe_stage_times")
    return {_lib.moe_stage_name(i).decode(): (tot[i], cnt[i]) for i in range(n)}
