"""Full-size K3 layers, run exactly as the benchmark times them (seeded inputs
generated on the device, QB on the batch from a zero bias, one workspace),
checked against the float64 oracle:

* router: the fp32 scores of sampled tokens against the oracle's router;
* routing: exact target loads, the top-k certificate (the selection is the
  top-k of the fixed-point biased scores under the returned bias) and the
  renormalised weights for every token; bit-exact indices, bias and QB
  counters against the oracle's QB on the same scores where the oracle
  finishes in seconds (T <= 4096);
* outputs: sampled tokens against the oracle layer on those tokens, with the
  oracle's weights computed from the same scores (experts decoded one at a
  time), max|diff| / rms(ref) within the bf16 / MXFP4 bounds.
"""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from layer_cases import announce, rel_err, w4a4_check
from oracle import layer as olayer
from oracle import qb

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "mxfp4": 1e-1, "mxfp4_a8": 1e-1, "mxfp4_a4": 1e-1}
SCALES = {"w_gate": "s_gate", "w_uproj": "s_uproj", "w_dn": "s_dn"}


def forward_as_benchmarked(shape, qb_mode, calls=1):
    import sparse_moe_ffn_sigmoid_amd as moe
    dev = torch.device("cuda:0")
    inp = workloads.layer_inputs(shape, dev, seed=0)
    w = {}
    for key, v in inp.items():
        if key == "x" or v is None:
            continue
        if isinstance(v, tuple):
            w[key], w[SCALES[key]] = v
        else:
            w[key] = v
    w["router_logit_offset"] = w.pop("logit_offset")
    routed = {"bf16": moe.MOE_BF16, "mxfp4": moe.MOE_MXFP4, "mxfp4_a8": moe.MOE_MXFP4_A8,
              "mxfp4_a4": moe.MOE_MXFP4_A4}[shape.routed]
    sh = moe.make_shape(shape.T, shape.d, shape.latent, shape.n, shape.k, shape.m, shape.shared,
                        moe.MOE_BF16, routed, shape.eps, qb_mode, 64)
    ws = torch.empty(moe.forward_workspace_bytes(sh), dtype=torch.uint8, device=dev)
    bias0 = torch.zeros(shape.n, dtype=torch.float64, device=dev)
    res = []
    for _ in range(calls):
        r = moe.latent_forward(sh, w, inp["x"], bias=bias0, workspace=ws, want_scores=True)
        torch.cuda.synchronize()
        res.append({k: v.float().cpu().numpy() if v.dtype == torch.bfloat16 else v.cpu().numpy()
                    for k, v in r.items()})
    return (inp, res[0]) if calls == 1 else (inp, res)


def check_routing(shape, got, qb_mode):
    s = got["scores"]
    T, n, k = s.shape[0], shape.n, shape.k
    # the selection is the top-k of the fixed-point biased keys (ties to the lower index)
    sfx = qb.to_fixed(s)
    bfx = np.rint(got["bias"] * 2.0 ** 40).astype(np.int64)
    assert (bfx.astype(np.float64) * 2.0 ** -40 == got["bias"]).all()
    key = qb.packed_keys(sfx, bfx)
    top = np.argpartition(-key, k - 1, axis=1)[:, :k]
    assert (np.sort(top, 1) == np.sort(got["idx"], 1)).all()
    # ordered by raw score, weights = chosen raw scores renormalised
    chosen = np.take_along_axis(s.astype(np.float64), got["idx"].astype(np.int64), 1)
    assert (np.diff(chosen, axis=1) <= 0).all()
    w_ref = chosen / chosen.sum(1, keepdims=True)
    assert np.abs(got["w"] - w_ref).max() <= (k + 1) * 2.0 ** -24
    if qb_mode == qb.MODE_BATCH:
        assert (got["loads"] == qb.targets(T, n, k)).all()
        assert got["info"][1] == qb.STATUS_OK
        if T <= 4096:
            ref = qb.route_qb(s, k)
            assert (got["idx"] == ref["idx"]).all()
            assert (got["bias"] == ref["bias"]).all()
            assert tuple(int(v) for v in got["info"]) == tuple(ref["info"])
    else:
        assert (bfx == 0).all()
        assert (got["loads"] == np.bincount(got["idx"].ravel(), minlength=n)).all()
    return w_ref


# last: how many experts (evenly spread, the first and last included) get
# the token in their last row slot sampled (the ragged end of their row
# group); None: every expert.  cover: tokens added until every expert is
# in the sample.  The decode batch is sampled whole (every expert it
# touches, every last row).
@pytest.mark.parametrize("wl,qb_mode,last,cover", [
    ("k3_decode", qb.MODE_BATCH, None, True),
    ("k3_prefill", qb.MODE_BATCH, 16, True),
    ("k3_mxfp4", qb.MODE_BATCH, 6, False),
    ("k3_mxfp4", qb.MODE_FROZEN, 6, False),
    ("k3_prefill_16k", qb.MODE_BATCH, 16, True),
    ("k3_mxfp4_a8", qb.MODE_BATCH, 6, False),
    ("k3_mxfp4_a4", qb.MODE_BATCH, 6, False),
])
def test_full_size_layer_sampled(wl, qb_mode, last, cover):
    check_sampled(workloads.SHAPES[wl], qb_mode, wl, last=last, cover=cover)


def test_forward_deterministic_k3_prefill():
    """Two calls on the same inputs and workspace give bitwise-equal results
    (no atomics decide an output value or its order)."""
    announce("determinism k3_prefill")
    inp, (a, b) = forward_as_benchmarked(workloads.SHAPES["k3_prefill"], qb.MODE_BATCH, calls=2)
    for key in a:
        assert a[key].dtype == b[key].dtype
        assert np.array_equal(a[key].view(np.uint8), b[key].view(np.uint8)), key
    del inp
    torch.cuda.empty_cache()


# K3 widths with fewer experts, so that each expert holds 150, 300 or 512 rows:
# one 160-row tile, one 320-row tile (ragged), two 256 x 256 tiles.
@pytest.mark.parametrize("T,n", [(600, 64), (1200, 64), (2048, 64)])
def test_tall_expert_tiles_k3_width(T, n):
    shape = dataclasses.replace(workloads.SHAPES["k3_prefill"], T=T, n=n)
    check_sampled(shape, qb.MODE_BATCH, f"T={T} n={n}", last=None)


def last_slot_tokens(idx, n):
    """For every expert, the last token routed to it (the token in the last
    row of the expert's row group, rows being filled in token order); -1
    for experts with no token."""
    T, k = idx.shape
    last = np.full(n, -1, np.int64)
    np.maximum.at(last, idx.ravel().astype(np.int64), np.repeat(np.arange(T), k))
    return last


def expert_cover(idx, tokens):
    """Greedy set cover: tokens added until every expert that received a
    token appears in some sampled token's selection."""
    T, k = idx.shape
    need = set(np.unique(idx).tolist()) - set(np.unique(idx[tokens]).tolist())
    chosen = list(tokens)
    while need:
        gain = np.array([len(need.intersection(row)) for row in idx.tolist()])
        t = int(np.argmax(gain))
        chosen.append(t)
        need -= set(idx[t].tolist())
    return chosen


def sampled_tokens(T, idx, n, last, cover=False):
    """First, thirds and last token; the tokens in the last row slot of
    `last` experts (evenly spread, first and last expert included; None:
    every expert); with `cover`, a greedy cover of every touched expert."""
    tokens = [0, T // 3, (2 * T) // 3, T - 1]
    lt = last_slot_tokens(idx, n)
    experts = np.arange(n) if last is None else np.unique(np.linspace(0, n - 1, last).astype(int))
    tokens += [int(t) for t in lt[experts] if t >= 0]
    if cover:
        tokens = expert_cover(idx, tokens)
    return np.unique(np.array(tokens))


def check_sampled(shape, qb_mode, name, last=4, cover=False):
    announce(f"layer {name} qb_mode={qb_mode}")
    inp, got = forward_as_benchmarked(shape, qb_mode)
    T = shape.T
    tokens = sampled_tokens(T, got["idx"], shape.n, last, cover)
    touched = np.unique(got["idx"][tokens])
    print(f"  {tokens.size} tokens sampled, {touched.size} experts", flush=True)
    if cover or last is None:
        assert touched.size == int((got["loads"] > 0).sum())
    # router on the sampled tokens
    x_s = olayer.as_f64(inp["x"][torch.from_numpy(tokens).cuda()])
    s_ref = olayer.router_scores(x_s, olayer.as_f64(inp["w_router"]),
                                 olayer.as_f64(inp["logit_offset"]))
    assert np.abs(got["scores"][tokens] - s_ref).max() <= 1e-5
    w_ref = check_routing(shape, got, qb_mode)
    # layer outputs of the sampled tokens, oracle weights from the same scores
    sub = dict(inp)
    sub["x"] = inp["x"][torch.from_numpy(tokens).cuda()]
    out_ref = olayer.layer_forward(sub, got["idx"][tokens], w_ref[tokens], shape.eps,
                                   act_mxfp8=shape.routed == "mxfp4_a8",
                                   act_mxfp4=shape.routed == "mxfp4_a4")
    err = rel_err(got["out"][tokens], out_ref)
    print(f"  info={got['info'].tolist()} sampled max|diff|/rms = {err:.3e}", flush=True)
    if shape.routed == "mxfp4_a4":
        w4a4_check(sub, got["idx"][tokens], w_ref[tokens], shape.eps, got["out"][tokens], out_ref,
                   TOL[shape.routed])
    else:
        assert err <= TOL[shape.routed]
    del inp, sub
    torch.cuda.empty_cache()
