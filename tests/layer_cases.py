"""Shared helpers of the layer parity tests (inputs, binding calls, metrics)."""
import sys

import numpy as np
import torch

import workloads
from oracle import layer as olayer
from oracle import qb

DT = {"f32": 0, "bf16": 1, "mxfp4": 2, "mxfp4_a8": 3}


def announce(name):
    print(f"\n[gpu case] {name}", flush=True)
    sys.stdout.flush()


def to_device(inp, dev="cuda"):
    """Generator output -> the binding's weight dict on the device."""
    w = {}
    for key, v in inp.items():
        if key == "x" or v is None:
            continue
        if isinstance(v, tuple):
            codes, scales = v
            w[key] = codes.to(dev)
            w[{"w_gate": "s_gate", "w_uproj": "s_uproj", "w_dn": "s_dn"}[key]] = scales.to(dev)
        else:
            w[key] = v.to(dev)
    return inp["x"].to(dev), w


def make_shape(moe, shape, T=None, qb_mode=1):
    T = shape.T if T is None else T
    return moe.make_shape(T, shape.d, shape.latent, shape.n, shape.k, shape.m, shape.shared,
                          DT[shape.act], DT[shape.routed], shape.eps, qb_mode, 64)


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.abs(got - ref).max() / np.sqrt(np.mean(ref * ref)))


def oracle_scores(inp):
    return olayer.router_scores(olayer.as_f64(inp["x"]), olayer.as_f64(inp["w_router"]),
                                None if inp.get("logit_offset") is None
                                else olayer.as_f64(inp["logit_offset"]))


def run_gpu(moe, shape, inp, scores_in=None, bias=None, qb_mode=1, T=None):
    x, w = to_device(inp)
    if "logit_offset" in inp and inp["logit_offset"] is not None:
        w["router_logit_offset"] = w.pop("logit_offset")
    sh = make_shape(moe, shape, T=T, qb_mode=qb_mode)
    s_in = None if scores_in is None else torch.from_numpy(scores_in).cuda()
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float64)).cuda()
    r = moe.latent_forward(sh, w, x, bias=b, scores_in=s_in, want_scores=True)
    torch.cuda.synchronize()
    out = {k: v.float().cpu().numpy() if v.dtype == torch.bfloat16 else v.cpu().numpy()
           for k, v in r.items()}
    return out
