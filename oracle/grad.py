"""Gradients of the Stable LatentMoE layer -- oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).  The layer's forward
pass written again with float64 PyTorch CPU tensors and differentiated by
autograd; the numbers are pinned against finite differences of
:func:`oracle.layer.layer_forward` (an independent NumPy implementation) in
the tests.

What is differentiated (the backward pass a training step needs; the pages
describe the forward layer, and [K3-structure-5] Q&A on routing fixes what
carries a gradient):

* The expert selection is held fixed: the QB bias acts on selection only and
  top-k is piecewise constant, so no gradient flows through the bias or the
  choice of experts.
* The mixture weights w = s_sel / sum(s_sel) are the chosen *raw* sigmoid
  scores renormalised, so the router weights, the logit offset and x receive
  gradients through them.
* Everything after routing is smooth: latent down-projection, SiTU-GLU
  experts (softcap tanh on gate and up), the weighted sum, RMSNorm with gain
  gamma, up-projection and the merged shared MLP.

Routed experts are dense (bf16-valued) matrices; MXFP4 weights are a
deployment format and are not trained here.

:func:`sgd_step` is the optimizer step that completes a training step: the
pages name no optimizer for the layer's weights (the Kimi K3 pages' Per-Head
Muon is outside this layer), so the plainest one, w <- w - lr * g, as
stated fp32 operations (each rounded to nearest even) stored in the
weight's own type.
"""
from __future__ import annotations

import numpy as np

from . import layer

GRAD_KEYS = ("x", "w_router", "logit_offset", "w_down", "w_up", "w_gate", "w_uproj", "w_dn",
             "rms_gamma", "ws_gate", "ws_up", "ws_down")


def _softcap(v, beta):
    import torch
    return beta * torch.tanh(v / beta)


def _situ(g, u):
    import torch
    gc = _softcap(g, layer.BETA_GATE)
    return gc * torch.sigmoid(gc) * _softcap(u, layer.BETA_UP)


def layer_grads(inp, idx, eps, dout):
    """Gradients of sum(out * dout) for the layer with the selection ``idx``
    [T, k] held fixed.  ``inp`` as for :func:`oracle.layer.layer_forward`
    (dense routed experts), ``dout`` [T, d].  Returns a dict of float64
    NumPy arrays keyed by :data:`GRAD_KEYS` (``logit_offset`` is None when
    the layer has no offset) and the forward output under ``"out"``."""
    import torch

    def leaf(a):
        return torch.tensor(layer.as_f64(a), dtype=torch.float64, requires_grad=True)

    P = {key: leaf(inp[key]) for key in GRAD_KEYS
         if key != "logit_offset" and inp.get(key) is not None}
    off = inp.get("logit_offset")
    P["logit_offset"] = leaf(off) if off is not None else None
    x = P["x"]
    T = x.shape[0]
    idx_t = torch.from_numpy(np.asarray(idx, np.int64))
    logits = x @ P["w_router"].T
    if P["logit_offset"] is not None:
        logits = logits + P["logit_offset"][None, :]
    s = torch.sigmoid(logits)
    s_sel = torch.gather(s, 1, idx_t)
    w = s_sel / s_sel.sum(dim=1, keepdim=True)
    z = x @ P["w_down"].T
    y = torch.zeros((T, z.shape[1]), dtype=torch.float64)
    idx_np = np.asarray(idx)
    for e in np.unique(idx_np):
        rows, slots = np.nonzero(idx_np == e)
        rows_t = torch.from_numpy(rows)
        ze = z[rows_t]
        h = _situ(ze @ P["w_gate"][int(e)].T, ze @ P["w_uproj"][int(e)].T)
        ye = (h @ P["w_dn"][int(e)].T) * w[rows_t, torch.from_numpy(slots)][:, None]
        y = y.index_add(0, rows_t, ye)
    yn = y / torch.sqrt(torch.mean(y * y, dim=1, keepdim=True) + eps) * P["rms_gamma"]
    out = yn @ P["w_up"].T
    hs = _situ(x @ P["ws_gate"].T, x @ P["ws_up"].T)
    out = out + hs @ P["ws_down"].T
    out.backward(torch.from_numpy(layer.as_f64(dout)))
    res = {key: (None if P[key] is None else P[key].grad.numpy()) for key in GRAD_KEYS}
    res["out"] = out.detach().numpy()
    return res


def sgd_step(w, g, lr, dtype):
    """One gradient-descent step on one weight tensor: t = fp32(lr * g), then
    fp32(w - t), each rounded to nearest even (IEEE single precision, no
    fused multiply-add), then stored as ``dtype`` ("f32", or "bf16" rounded
    to nearest even).  Returns float64 values of the stored result."""
    w32 = np.asarray(layer.as_f64(w), np.float64).astype(np.float32)
    g32 = np.asarray(layer.as_f64(g), np.float64).astype(np.float32)
    t = np.multiply(np.float32(lr), g32, dtype=np.float32)
    r = np.subtract(w32, t, dtype=np.float32)
    if dtype == "bf16":
        return layer.bf16_round(r.astype(np.float64))
    return r.astype(np.float64)
