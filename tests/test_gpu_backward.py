"""Parity of moe_latent_backward (HIP) with the float64 gradient oracle.

Protocol: the HIP forward runs on the oracle's fp32 router scores
(``scores_in``); its routing (idx, w) and those scores feed the HIP backward,
and the same selection feeds the oracle (which recomputes the mixture
weights from the exact scores).  Every gradient tensor is compared as
max|diff| / rms(ref) against the bound below; experts and router rows that
no token chose must receive exactly zero.
"""
import numpy as np
import pytest
import torch

import workloads
from layer_cases import announce, oracle_scores, rel_err, to_device, make_shape
from oracle import grad as ograd
from oracle import layer as olayer

pytestmark = pytest.mark.gpu

# Bounds, derived from the arithmetic.  Every gradient entry is a sum of
# products whose factors went through a few bf16 roundings (relative 2^-9
# each): the recomputed z, h, h_s and yhat, and the intermediate gradients
# that feed a product (dy per slot, dg, du, dgs, dus, dz).  With at most four
# roundings along a term, each term is off by at most 4 * 2^-9 = 0.8%, and
# independent roundings make the relative Frobenius error of a whole tensor
# about 2^-9 * sqrt(4) = 0.4%: TOL_FRO = 1e-2.  A row (one token of dx, one
# expert of a stacked expert gradient, one output row of a weight gradient)
# can be a sum of very few terms with cancellation between them (a router
# row fed by a single token), so rows get TOL_ROW = 1e-1, still far below
# the O(1) error of a wrong row, tile or expert.  The roundings are relative
# to the terms, not to their sum: a router row fed by one token is that
# token's dlogit times x, and dlogit is dw_j minus the weighted mean of the
# token's dw, so when the two nearly cancel the row's relative error has no
# bound while its absolute error stays at the scale of the terms, about the
# same for every row.  A row is therefore measured against ROW_FLOOR = 25% of
# the median row norm of its tensor when its own norm is smaller (absolute
# error <= 2.5% of the median, about six times the 0.4% a term carries).
# Elementwise max|diff| / rms is printed but not bounded: rounding z and h to
# bf16 alone moves a rank-one expert gradient (one token per expert) by 12%
# of its rms at its largest entries.
TOL_FRO = 1e-2
TOL_ROW = 1e-1
ROW_FLOOR = 0.25


def worst_row(got, ref):
    """max over rows of |got - ref| / max(|ref|, ROW_FLOOR * median row norm);
    rows of an all-zero reference (experts no token chose) are skipped."""
    gg, rr = got.reshape(ref.shape[0], -1), ref.reshape(ref.shape[0], -1)
    nr = np.linalg.norm(rr, axis=1)
    ok = nr > 0
    if not ok.any():
        return 0.0
    floor = ROW_FLOOR * float(np.median(nr[ok]))
    return float((np.linalg.norm(gg - rr, axis=1)[ok] / np.maximum(nr[ok], floor)).max())

KEYS = {"dx": "x", "d_w_router": "w_router", "d_router_logit_offset": "logit_offset",
        "d_w_down": "w_down", "d_w_up": "w_up", "d_w_gate": "w_gate", "d_w_uproj": "w_uproj",
        "d_w_dn": "w_dn", "d_rms_gamma": "rms_gamma", "d_ws_gate": "ws_gate", "d_ws_up": "ws_up",
        "d_ws_down": "ws_down"}


def check_backward(shape, seed, name):
    import sparse_moe_ffn_sigmoid_amd as moe
    announce(f"backward {name} {shape}")
    inp = workloads.layer_inputs(shape, "cpu", seed=seed, random_gamma=True)
    s = oracle_scores(inp)
    x, w = to_device(inp)
    w["router_logit_offset"] = w.pop("logit_offset", None)
    sh = make_shape(moe, shape)
    fwd = moe.latent_forward(sh, w, x, scores_in=torch.from_numpy(s).cuda(), want_scores=True)
    rng = np.random.default_rng(seed + 1)
    dout = torch.from_numpy(rng.standard_normal((shape.T, shape.d)).astype(np.float32)).to(
        torch.bfloat16)
    got = moe.latent_backward(sh, w, x, fwd["scores"], fwd["idx"], fwd["w"], dout.cuda())
    torch.cuda.synchronize()
    idx = fwd["idx"].cpu().numpy()
    ref = ograd.layer_grads(inp, idx, shape.eps, dout.double().numpy())
    unused = np.setdiff1d(np.arange(shape.n), np.unique(idx))
    worst = 0.0
    for gname, key in KEYS.items():
        g = got[gname]
        if g is None:
            assert ref[key] is None
            continue
        gv = g.float().cpu().numpy()
        r = ref[key]
        fro = float(np.linalg.norm(gv - r) / np.linalg.norm(r))
        row = worst_row(gv, r) if r.ndim >= 2 else fro
        worst = max(worst, fro)
        print(f"  {gname:<24} rel. Frobenius {fro:.2e}, worst row {row:.2e}, "
              f"max|diff|/rms {rel_err(gv, r):.2e}", flush=True)
        assert fro <= TOL_FRO and row <= TOL_ROW, (gname, fro, row)
        if gname in ("d_w_gate", "d_w_uproj", "d_w_dn", "d_w_router") and unused.size:
            assert (gv[unused] == 0).all()
    return worst


@pytest.mark.parametrize("kw", [
    dict(T=200),                                              # several tiles, ragged rows
    dict(T=37, n=24, k=3, d=448, latent=192, m=128, shared=192),
    dict(T=16, n=64, k=4),                                    # ~1 row per expert, unused experts
    dict(T=1000, n=16, k=4, seed=7),                          # 250 rows per expert
    dict(T=584, n=64, k=8, seed=4),                           # 73 rows: the 96-row tiles
])
def test_bf16_backward(kw):
    kw = dict(kw)
    seed = kw.pop("seed", 1)
    check_backward(workloads.small_shape(**kw), seed, f"bf16 {kw}")


def test_backward_k3_widths():
    """d = 7168, latent 3584, inter 2048, shared 6144, k = 16 with 64 experts
    (150 rows each): the tile configurations of the K3 shapes."""
    import dataclasses
    shape = dataclasses.replace(workloads.SHAPES["k3_prefill"], T=600, n=64)
    check_backward(shape, 5, "K3 widths, 64 experts")


def test_backward_without_logit_offset():
    check_backward(workloads.small_shape(T=120, offset_std=0.0), 3, "no offset")


def test_backward_deterministic():
    import sparse_moe_ffn_sigmoid_amd as moe
    shape = workloads.small_shape(T=300, n=16, k=4)
    inp = workloads.layer_inputs(shape, "cpu", seed=2, random_gamma=True)
    x, w = to_device(inp)
    w["router_logit_offset"] = w.pop("logit_offset")
    sh = make_shape(moe, shape)
    fwd = moe.latent_forward(sh, w, x, want_scores=True)
    dout = torch.randn((shape.T, shape.d), generator=torch.Generator().manual_seed(0)).to(
        torch.bfloat16).cuda()
    a = moe.latent_backward(sh, w, x, fwd["scores"], fwd["idx"], fwd["w"], dout)
    b = moe.latent_backward(sh, w, x, fwd["scores"], fwd["idx"], fwd["w"], dout)
    torch.cuda.synchronize()
    for key in a:
        if a[key] is not None:
            assert torch.equal(a[key].view(torch.uint8) if a[key].dtype == torch.bfloat16
                               else a[key], b[key].view(torch.uint8)
                               if b[key].dtype == torch.bfloat16 else b[key]), key


@pytest.mark.parametrize("saved", [False, True])
def test_backward_k3_prefill_full_size_dx_sampled(saved):
    """The full K3 prefill layer (T = 4096, 896 experts, k = 16), forward and
    backward as the benchmark runs them (saved: the training forward keeps
    its activations and the backward reads them); dx of sampled tokens
    (first, thirds, last and the last token of the first and last expert)
    against the gradient oracle on each token alone.  Tokens are independent
    once the selection is fixed, so a token's dx needs only its own 16
    experts: the oracle runs on the token with those experts' weights
    (router rows, gate, up, down) and the full dense weights."""
    import sparse_moe_ffn_sigmoid_amd as moe
    shape = workloads.SHAPES["k3_prefill"]
    announce(f"backward full size {shape}")
    dev = torch.device("cuda:0")
    inp = workloads.layer_inputs(shape, dev, seed=0)
    w = {key: v for key, v in inp.items() if key != "x" and v is not None}
    w["router_logit_offset"] = w.pop("logit_offset")
    sh = moe.make_shape(shape.T, shape.d, shape.latent, shape.n, shape.k, shape.m, shape.shared,
                        moe.MOE_BF16, moe.MOE_BF16, shape.eps, moe.MOE_QB_BATCH, 64)
    sv = (torch.empty(moe.saved_activations_bytes(sh), dtype=torch.uint8, device=dev)
          if saved else None)
    fwd = moe.latent_forward(sh, w, inp["x"], want_scores=True, saved=sv)
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    dout = torch.randn(inp["x"].shape, generator=g, device=dev, dtype=torch.float32).to(
        torch.bfloat16)
    if saved:
        got = moe.latent_backward_train(sh, w, inp["x"], fwd["scores"], fwd["idx"], fwd["w"],
                                        dout, sv)
    else:
        got = moe.latent_backward(sh, w, inp["x"], fwd["scores"], fwd["idx"], fwd["w"], dout)
    torch.cuda.synchronize()
    idx = fwd["idx"].cpu().numpy()
    dx = got["dx"].float().cpu().numpy()
    del got, sv
    torch.cuda.empty_cache()
    T = shape.T
    flat = idx.ravel()
    tokens = [0, T // 3, (2 * T) // 3, T - 1,
              int(np.nonzero(flat == idx.min())[0].max()) // shape.k,
              int(np.nonzero(flat == idx.max())[0].max()) // shape.k]
    dense = {key: olayer.as_f64(inp[key]) for key in ("w_down", "w_up", "rms_gamma", "ws_gate",
                                                       "ws_up", "ws_down")}
    ref_rows, got_rows = [], []
    for t in sorted(set(tokens)):
        sel = torch.from_numpy(idx[t].astype(np.int64)).to(dev)
        sub = dict(dense)
        sub["x"] = olayer.as_f64(inp["x"][t:t + 1])
        for key in ("w_router", "logit_offset", "w_gate", "w_uproj", "w_dn"):
            sub[key] = olayer.as_f64(inp[key][sel])
        ref = ograd.layer_grads(sub, np.arange(shape.k)[None, :], shape.eps,
                                dout[t:t + 1].double().cpu().numpy())
        ref_rows.append(ref["x"][0])
        got_rows.append(dx[t])
        row = float(np.linalg.norm(dx[t] - ref["x"][0]) / np.linalg.norm(ref["x"][0]))
        print(f"  token {t}: dx rel. error {row:.2e}", flush=True)
        assert row <= TOL_ROW
    r, gv = np.stack(ref_rows), np.stack(got_rows)
    fro = float(np.linalg.norm(gv - r) / np.linalg.norm(r))
    print(f"  sampled dx rel. Frobenius {fro:.2e}", flush=True)
    assert fro <= TOL_FRO
    del inp, fwd, dout
    torch.cuda.empty_cache()
