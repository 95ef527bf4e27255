"""Seeded synthetic inputs for the Stable LatentMoE layer.

This module only draws random numbers and packs them into the layouts the
layer consumes; it holds none of the layer's arithmetic (no router, no
activation, no normalisation, no decoding of MXFP4 codes).  Both the HIP path
and the oracle take their inputs from here and nothing else is shared between
them.

Shapes and distributions (per workload):

* ``tiny``          T=64, d=256, latent 128, n=32, k=4, m=64, shared 2x64,
                    fp32 throughout; x~N(0,1), weights~N(0,1/fan_in), router
                    W~N(0,0.02^2); no logit offset.
* ``qb``            T=57344, n=896, k=16: router logits = N(0,1) + per-expert
                    popularity offset p_e~N(0,0.5^2) (routing only).
* ``k3_prefill``    T=4096, d=7168, latent 3584, n=896, k=16, m=2048, shared
                    2x3072; bf16 activations and weights, fp32 router
                    W~N(0,1/d) and offset p_e~N(0,0.5^2).
* ``k3_decode``     as k3_prefill with T=64.
* ``k3_mxfp4``      as k3_prefill with T=16384, routed experts in MXFP4
                    (OCP microscaling: E2M1 elements, one E8M0 scale per 32
                    consecutive K elements), p_e~N(0,1).

Random streams: torch generators seeded per (seed, tensor id, chunk), so
every tensor -- and every chunk of expert weights -- can be regenerated on
its own, on the CPU or on a GPU (the two devices give different but each
deterministic streams).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class LayerShape:
    T: int
    d: int
    latent: int
    n: int
    k: int
    m: int
    shared: int            # merged shared-expert intermediate width
    act: str               # "f32" | "bf16"
    routed: str            # "f32" | "bf16" | "mxfp4" | "mxfp4_a8" | "mxfp4_a4" (same weights
                           # as mxfp4)
    router_std: float      # std of the router weights
    offset_std: float      # std of the per-expert logit offset (0: none)
    eps: float = 1e-6


SHAPES = {
    "tiny": LayerShape(64, 256, 128, 32, 4, 64, 128, "f32", "f32", 0.02, 0.0),
    "k3_prefill": LayerShape(4096, 7168, 3584, 896, 16, 2048, 6144, "bf16", "bf16",
                             7168 ** -0.5, 0.5),
    "k3_decode": LayerShape(64, 7168, 3584, 896, 16, 2048, 6144, "bf16", "bf16",
                            7168 ** -0.5, 0.5),
    "k3_mxfp4": LayerShape(16384, 7168, 3584, 896, 16, 2048, 6144, "bf16", "mxfp4",
                           7168 ** -0.5, 1.0),
    # the MXFP4 batch with the routed experts' activations in MXFP8 (W4A8)
    "k3_mxfp4_a8": LayerShape(16384, 7168, 3584, 896, 16, 2048, 6144, "bf16", "mxfp4_a8",
                              7168 ** -0.5, 1.0),
    # ... and in MXFP4 (W4A4)
    "k3_mxfp4_a4": LayerShape(16384, 7168, 3584, 896, 16, 2048, 6144, "bf16", "mxfp4_a4",
                              7168 ** -0.5, 1.0),
    # the bf16 prefill layer at 16384 tokens: compute-bound (MFMA) instead of
    # bound by streaming the routed weights
    "k3_prefill_16k": LayerShape(16384, 7168, 3584, 896, 16, 2048, 6144, "bf16", "bf16",
                                 7168 ** -0.5, 0.5),
}

QB_SHAPE = dict(T=57344, n=896, k=16, offset_std=0.5)

# tensor ids of the random streams
_IDS = dict(x=1, w_router=2, offset=3, w_down=4, w_up=5, w_gate=6, w_uproj=7,
            w_dn=8, gamma=9, ws_gate=10, ws_up=11, ws_down=12, logits=13)
EXPERT_CHUNK = 32


def _gen(device, seed: int, tensor: str, chunk: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 64 + _IDS[tensor]) << 20) + chunk)
    return g


def normal(shape, std, device, seed, tensor, chunk=0, dtype=torch.float32):
    g = _gen(device, seed, tensor, chunk)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def qb_logits(T, n, offset_std, seed=0):
    """Router logits for the routing-only workload, NumPy PCG64 (float32):
    N(0,1) per (token, expert) plus a per-expert offset N(0, offset_std^2)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(2,))))
    p = rng.standard_normal(n, dtype=np.float32) * np.float32(offset_std)
    z = rng.standard_normal((T, n), dtype=np.float32)
    z += p[None, :]
    return z


# --------------------------------------------------------------------------
# MXFP4 (OCP Microscaling v1.0, E2M1 elements, E8M0 block scale, block 32)
# --------------------------------------------------------------------------
# Rounding thresholds on |v| / 2^E for the eight E2M1 magnitude codes
# 0, 0.5, 1, 1.5, 2, 3, 4, 6 (codes 0..7), ties to the even code; values at
# or above 6 saturate to code 7.
_E2M1_UPPER = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
_E2M1_TIE_UP = (False, True, False, True, False, True, False)


def mxfp4_quantize(w: torch.Tensor):
    """Quantise ``w`` [rows, K] (K % 32 == 0) to MXFP4.

    Returns (codes uint8 [rows, K/2], scales uint8 [rows, K/32]).  Element
    2i sits in the low nibble of byte i, element 2i+1 in the high nibble; bit
    3 of a nibble is the sign.  Block scale exponent = floor(log2(amax)) - 2
    (the largest E2M1 exponent), stored biased by 127 and clamped to
    [0, 254]; an all-zero block stores 0.
    """
    rows, K = w.shape
    assert K % 32 == 0
    wb = w.float().reshape(rows, K // 32, 32)
    amax = wb.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax.clamp_min(1e-38))) - 2,
                    torch.full_like(amax, -127.0))
    e = e.clamp(-127, 127)
    scales = (e + 127).to(torch.uint8)
    a = (wb.abs() / torch.exp2(e)[..., None])
    code = torch.zeros_like(a, dtype=torch.uint8)
    for i, (thr, up) in enumerate(zip(_E2M1_UPPER, _E2M1_TIE_UP)):
        above = (a >= thr) if up else (a > thr)
        code += above.to(torch.uint8)
    code |= (wb < 0).to(torch.uint8) << 3
    code = code.reshape(rows, K)
    codes = (code[:, 0::2] | (code[:, 1::2] << 4)).contiguous()
    return codes, scales.reshape(rows, K // 32).contiguous()


# --------------------------------------------------------------------------
# Layer inputs
# --------------------------------------------------------------------------
def _expert_weights(name, n, rows, cols, std, dtype, device, seed, mxfp4):
    """[n, rows, cols] expert weights, generated EXPERT_CHUNK experts at a time."""
    if mxfp4:
        codes = torch.empty((n, rows, cols // 2), dtype=torch.uint8, device=device)
        scales = torch.empty((n, rows, cols // 32), dtype=torch.uint8, device=device)
    else:
        out = torch.empty((n, rows, cols), dtype=dtype, device=device)
    for c, e0 in enumerate(range(0, n, EXPERT_CHUNK)):
        e1 = min(n, e0 + EXPERT_CHUNK)
        w = normal((e1 - e0, rows, cols), std, device, seed, name, c)
        if mxfp4:
            q, s = mxfp4_quantize(w.reshape(-1, cols))
            codes[e0:e1] = q.reshape(e1 - e0, rows, cols // 2)
            scales[e0:e1] = s.reshape(e1 - e0, rows, cols // 32)
        else:
            out[e0:e1] = w.to(dtype)
        del w
    return (codes, scales) if mxfp4 else out


def layer_inputs(shape: LayerShape, device="cpu", seed=0, random_gamma=False, T=None):
    """All inputs of one layer call as torch tensors on ``device``.

    Activations and dense weights use ``shape.act`` precision (fp32 or bf16,
    rounded to nearest even from fp32 draws); the router weights, the logit
    offset and the RMSNorm gain are fp32; routed experts use ``shape.routed``
    (MXFP4 gives ``w_gate``/``w_uproj``/``w_dn`` as (codes, scales) pairs).
    """
    T = shape.T if T is None else T
    adt = torch.float32 if shape.act == "f32" else torch.bfloat16
    rdt = torch.float32 if shape.routed == "f32" else torch.bfloat16
    mx = shape.routed in ("mxfp4", "mxfp4_a8", "mxfp4_a4")
    d, l, n, m, ms = shape.d, shape.latent, shape.n, shape.m, shape.shared
    inp = dict(
        x=normal((T, d), 1.0, device, seed, "x", dtype=adt),
        w_router=normal((n, d), shape.router_std, device, seed, "w_router"),
        logit_offset=(normal((n,), shape.offset_std, device, seed, "offset")
                      if shape.offset_std > 0 else None),
        w_down=normal((l, d), d ** -0.5, device, seed, "w_down", dtype=adt),
        w_up=normal((d, l), l ** -0.5, device, seed, "w_up", dtype=adt),
        w_gate=_expert_weights("w_gate", n, m, l, l ** -0.5, rdt, device, seed, mx),
        w_uproj=_expert_weights("w_uproj", n, m, l, l ** -0.5, rdt, device, seed, mx),
        w_dn=_expert_weights("w_dn", n, l, m, m ** -0.5, rdt, device, seed, mx),
        rms_gamma=(0.5 + torch.rand((l,), generator=_gen(device, seed, "gamma"),
                                    device=device) if random_gamma
                   else torch.ones((l,), device=device)),
        ws_gate=normal((ms, d), d ** -0.5, device, seed, "ws_gate", dtype=adt),
        ws_up=normal((ms, d), d ** -0.5, device, seed, "ws_up", dtype=adt),
        ws_down=normal((d, ms), ms ** -0.5, device, seed, "ws_down", dtype=adt),
    )
    return inp


def small_shape(**kw) -> LayerShape:
    """A reduced layer for fast parity tests (defaults: bf16, several tiles
    and a ragged tail in every dimension)."""
    base = dict(T=200, d=512, latent=256, n=40, k=6, m=192, shared=320, act="bf16",
                routed="bf16", router_std=512 ** -0.5, offset_std=0.5)
    base.update(kw)
    return LayerShape(**base)
