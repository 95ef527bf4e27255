"""Shared helpers of the layer parity tests (inputs, binding calls, metrics)."""
import sys

import numpy as np
import torch

import workloads
from oracle import layer as olayer
from oracle import qb

DT = {"f32": 0, "bf16": 1, "mxfp4": 2, "mxfp4_a8": 3, "mxfp4_a4": 4}


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


# --- W4A4: roundings that fp32 and float64 may take differently ------------
#
# The W4A4 experts read z and h as MXFP4 quantised from their bf16 storage.
# The kernel forms z and h in fp32 and the oracle in float64; where an exact
# value lies within the fp32 error of a bf16 rounding midpoint, both bf16
# neighbours are correct roundings, and with E2M1's coarse grid the choice can
# move that element by a whole E2M1 step or a block's shared exponent by one.
# A token whose output misses the bar is accepted when taking the other bf16
# neighbour of one such element (in z, or in h of one of its experts) brings
# it within the bar; everything else is compared as usual.

AMBIG_REL = 1e-5   # fp32 accumulation and transcendental error, with a wide margin


def _ambiguous(v):
    """Indices of elements whose bf16 rounding is not decided at AMBIG_REL,
    and the other bf16 neighbour of each."""
    v = np.asarray(v, np.float64)
    lo = olayer.bf16_round(v * (1 - AMBIG_REL))
    hi = olayer.bf16_round(v * (1 + AMBIG_REL))
    b = olayer.bf16_round(v)
    idx = np.nonzero(lo != hi)[0]
    other = np.where(lo[idx] != b[idx], lo[idx], hi[idx])
    return idx, other


def _w4a4_token(inp, t, experts, weights, eps, z_flip=None, h_flip=None):
    """Layer output of token t (float64) with z and h rounded as the W4A4
    experts read them; z_flip = (i, value) and h_flip = (j, i, value) replace
    one bf16-rounded element by its other neighbour."""
    x = olayer.as_f64(inp["x"][t:t + 1])
    z = olayer.bf16_round((x @ olayer.as_f64(inp["w_down"]).T)[0])
    if z_flip is not None:
        z[z_flip[0]] = z_flip[1]
    zq = olayer.mxfp4_act_round(z[None, :])
    y = np.zeros(z.shape[0])
    hs = []
    for j, (e, wj) in enumerate(zip(experts, weights)):
        wg = olayer.expert_matrix(inp["w_gate"], int(e))
        wu = olayer.expert_matrix(inp["w_uproj"], int(e))
        wd = olayer.expert_matrix(inp["w_dn"], int(e))
        h_exact = olayer.situ_glu(zq @ wg.T, zq @ wu.T)[0]
        h = olayer.bf16_round(h_exact)
        if h_flip is not None and h_flip[0] == j:
            h[h_flip[1]] = h_flip[2]
        hs.append(h_exact)
        y += wj * (olayer.mxfp4_act_round(h[None, :]) @ wd.T)[0]
    out = olayer.rmsnorm(y[None, :], olayer.as_f64(inp["rms_gamma"]), eps) @ olayer.as_f64(inp["w_up"]).T
    out += olayer.shared_mlp(x, inp["ws_gate"], inp["ws_up"], inp["ws_down"])
    return out[0], z, hs


def w4a4_check(inp, idx, w, eps, got, ref, tol):
    """Per-token check of a W4A4 layer against the oracle, with the
    ambiguous bf16 roundings of z and h allowed as described above."""
    rms = float(np.sqrt(np.mean(np.asarray(ref, np.float64) ** 2)))
    per = np.abs(got - ref).max(axis=1) / rms
    bad = np.nonzero(per > tol)[0]
    print(f"  per-token max|diff|/rms: median {np.median(per):.3e}, "
          f"{bad.size} of {per.size} tokens above {tol}", flush=True)
    assert bad.size <= max(2, per.size // 200), "more tokens off than rounding ambiguity explains"
    for t in bad:
        base, z, hs = _w4a4_token(inp, int(t), idx[t], w[t], eps)
        assert np.abs(base - ref[t]).max() / rms < 1e-9      # the helper is the oracle's layer
        best = np.inf
        x = olayer.as_f64(inp["x"][t:t + 1])
        z_exact = (x @ olayer.as_f64(inp["w_down"]).T)[0]
        zi, zo = _ambiguous(z_exact)
        for i, v in zip(zi, zo):
            out, _, _ = _w4a4_token(inp, int(t), idx[t], w[t], eps, z_flip=(i, v))
            best = min(best, np.abs(got[t] - out).max() / rms)
        for j, h_exact in enumerate(hs):
            hi, ho = _ambiguous(h_exact)
            for i, v in zip(hi, ho):
                out, _, _ = _w4a4_token(inp, int(t), idx[t], w[t], eps, h_flip=(j, i, v))
                best = min(best, np.abs(got[t] - out).max() / rms)
        print(f"  token {t}: {per[t]:.3e}; {zi.size} ambiguous z, "
              f"{sum(_ambiguous(h)[0].size for h in hs)} ambiguous h elements; "
              f"best with one of them flipped {best:.3e}", flush=True)
        assert best <= tol
