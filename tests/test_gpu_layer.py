"""Parity of moe_latent_forward (HIP) with the float64 layer oracle.

Protocol ("identical scores"): the oracle's fp32 router scores are passed to
the HIP layer as ``scores_in``, so both sides route from the same numbers;
indices, loads, bias and QB counters must then match bit for bit and the
outputs within max|diff| / rms(ref) <= 2e-2 (bf16), 1e-1 (MXFP4 against the
oracle on the decoded weights) or 1e-4 (fp32).  The HIP router is checked
separately against the oracle's scores (max abs difference <= 1e-5).
"""
import numpy as np
import pytest

import workloads
from layer_cases import announce, oracle_scores, rel_err, run_gpu, w4a4_check
from oracle import layer as olayer
from oracle import qb

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "mxfp4": 1e-1, "mxfp4_a8": 1e-1, "mxfp4_a4": 1e-1}


def check_layer(shape, seed=0, qb_mode=qb.MODE_BATCH, bias=None, name="", edit=None):
    import sparse_moe_ffn_sigmoid_amd as moe
    announce(f"layer {name} {shape}")
    inp = workloads.layer_inputs(shape, "cpu", seed=seed, random_gamma=True)
    if edit is not None:
        edit(inp)
    s = oracle_scores(inp)
    ref = qb.route_qb(s, shape.k, bias=bias, mode=qb_mode)
    got = run_gpu(moe, shape, inp, scores_in=s, bias=bias, qb_mode=qb_mode)
    assert (got["idx"] == ref["idx"]).all()
    assert (got["loads"] == ref["loads"]).all()
    assert tuple(int(v) for v in got["info"]) == tuple(ref["info"])
    if qb_mode == qb.MODE_BATCH:
        assert (got["bias"] == ref["bias"]).all()
    out_ref = olayer.layer_forward(inp, ref["idx"], ref["w"], shape.eps,
                                   act_mxfp8=shape.routed == "mxfp4_a8",
                                   act_mxfp4=shape.routed == "mxfp4_a4")
    err = rel_err(got["out"], out_ref)
    print(f"  max|diff|/rms = {err:.3e}", flush=True)
    tol = TOL[shape.routed if shape.routed.startswith("mxfp4") else shape.act]
    if shape.routed == "mxfp4_a4":
        w4a4_check(inp, ref["idx"], ref["w"], shape.eps, got["out"], out_ref, tol)
    else:
        assert err <= tol, err
    # the HIP router on its own
    announce(f"router {name}")
    own = run_gpu(moe, shape, inp, bias=bias, qb_mode=qb_mode)
    assert np.abs(own["scores"] - s).max() <= 1e-5
    return got, ref


def test_fp32_layer_on_permutation_weights():
    """The HIP layer (fp32, frozen zero bias) on weights that are scaled
    permutation matrices, against the output written out by hand
    (``tests/perm_layer.py``); no oracle is involved."""
    import torch
    import perm_layer as P
    import sparse_moe_ffn_sigmoid_amd as moe
    inp, par = P.build()
    shape = workloads.small_shape(T=P.T, d=P.D, latent=P.LAT, n=P.N, k=P.K, m=P.LAT,
                                  shared=P.S, act="f32", routed="f32", eps=P.EPS)
    tin = {key: torch.from_numpy(np.ascontiguousarray(v, np.float32)) for key, v in inp.items()}
    announce("fp32 layer on permutation weights")
    got = run_gpu(moe, shape, tin, bias=np.zeros(P.N), qb_mode=qb.MODE_FROZEN)
    assert (got["idx"] == P.TOP).all()
    sc = 1.0 / (1.0 + np.exp(-P.LOGIT_OFFSET[P.TOP]))
    assert np.allclose(got["w"], (sc / sc.sum())[None, :], rtol=1e-6, atol=0)
    want = P.expected(inp, par, got["idx"], got["w"].astype(np.float64))
    err = rel_err(got["out"], want)
    print(f"  max|diff|/rms = {err:.3e}", flush=True)
    assert err <= TOL["f32"], err


def test_tiny_fp32_layer():
    check_layer(workloads.SHAPES["tiny"], name="tiny fp32")


@pytest.mark.parametrize("kw", [
    dict(),                                                   # several tiles, ragged rows
    dict(T=37, n=24, k=3, d=448, latent=192, m=128, shared=192),
    dict(T=16, n=64, k=4),                                     # ~1 row per expert (small-M tile)
    dict(T=500, n=16, k=2, latent=320),                        # 62-63 rows: one 96-row tile, column tails in both GEMMs
    dict(T=600, n=16, k=4),                                    # 150 rows per expert: one 160-row tile
    dict(T=1000, n=16, k=4, seed=7),                           # 250 rows: one 320-row tile (8 waves)
    dict(T=1200, n=16, k=4, d=512, seed=1),                    # 300 rows: one 320-row tile, ragged
    dict(T=1, n=64, k=4),                                      # one token: M = 1 everywhere
    dict(T=3, n=16, k=2),
])
def test_bf16_layer(kw):
    kw = dict(kw)
    seed = kw.pop("seed", 1)
    check_layer(workloads.small_shape(**kw), seed=seed, name=f"bf16 {kw}")


def test_mxfp4_layer():
    check_layer(workloads.small_shape(routed="mxfp4", T=300, k=4), seed=2, name="mxfp4 qb")


# Widths that are multiples of 512 take the pipelined MXFP4 kernel (scale
# panel in LDS); the others take the register-staged one, except for 161 -
# 320 rows per expert, where widths that are multiples of 128 take the
# 320-row kernel (8 waves, scales through the ring).  Cases cover the tile
# shapes (few rows per expert: 32 x 256; many: 160 x 256 and 320 x 256), row
# and column tails.
@pytest.mark.parametrize("kw", [
    dict(T=300, k=4, d=1024, latent=512, m=512),              # 32x256 tiles, both GEMMs
    dict(T=300, k=4, d=1024, latent=512, m=576),              # gate/up column tail
    dict(T=300, k=4, d=1024, latent=640, m=512),              # down column tail
    dict(T=640, n=16, k=4, d=1024, latent=512, m=512, shared=256),  # 160-row tiles, full
    dict(T=700, n=16, k=4, d=1024, latent=512, m=512, shared=256),  # one 320-row tile, 175 rows
    dict(T=1200, n=16, k=4, d=1024, latent=512, m=512, shared=256),  # one 320-row tile, 300 rows
    dict(T=1000, n=16, k=4, d=1024, latent=640, m=512, shared=256),  # 320 rows, 20 scale bytes per row
])
def test_mxfp4_layer_pipelined(kw):
    check_layer(workloads.small_shape(routed="mxfp4", **kw), seed=5, name=f"mxfp4 {kw}")


def extreme_scale_bytes(inp, seed=0):
    """Scale bytes at the ends of the E8M0 range: 0 and 1 (products below
    the normal bf16 range) on a tenth of the routed blocks, 253 and 254 on
    blocks whose codes are all zero (+0 or -0)."""
    rng = np.random.default_rng(seed)
    for key in ("w_gate", "w_uproj", "w_dn"):
        codes, scales = (t.clone() for t in inp[key])
        sc = scales.numpy()
        cd = codes.numpy()
        r = rng.random(sc.shape)
        sc[r < 0.1] = rng.integers(0, 2, size=int((r < 0.1).sum()))
        big = r > 0.97
        sc[big] = rng.integers(253, 255, size=int(big.sum()))
        blk = cd.reshape(*sc.shape, 16)
        blk[big] = rng.choice(np.array([0x00, 0x88, 0x08, 0x80], np.uint8), size=(int(big.sum()), 16))
        inp[key] = (codes, scales)


# Both MXFP4 decoders (bf16 by exponent arithmetic in the register-staged
# kernel, the hardware conversion in the pipelined one) over the whole E8M0
# byte range that a finite product allows
@pytest.mark.parametrize("kw", [
    dict(T=300, k=4),                                          # register-staged kernel
    dict(T=300, k=4, d=1024, latent=512, m=512),               # pipelined kernel, 32-row tiles
    dict(T=1200, n=16, k=4, d=1024, latent=512, m=512, shared=256),  # 320-row tiles
])
def test_mxfp4_layer_extreme_scale_bytes(kw):
    check_layer(workloads.small_shape(routed="mxfp4", **kw), seed=4,
                name=f"mxfp4 extreme scales {kw}", edit=extreme_scale_bytes)


def test_w4a8_layer_extreme_scale_bytes():
    shape = workloads.small_shape(routed="mxfp4_a8", T=300, n=16, k=4, d=1024, latent=512,
                                  m=512, shared=256)
    check_layer(shape, seed=4, name="w4a8 extreme scales", edit=extreme_scale_bytes)


# W4A8: MXFP4 weights times MXFP8 activations on the scaled MFMA (320-row
# tiles only), against the oracle that rounds z and h to bf16 and then MXFP8
@pytest.mark.parametrize("kw", [
    dict(T=300, n=16, k=4, d=1024, latent=512, m=512, shared=256),   # 75 rows per expert
    dict(T=1200, n=16, k=4, d=1024, latent=512, m=512, shared=256),  # 300 rows per expert
    dict(T=1000, n=16, k=4, d=1024, latent=640, m=384, shared=256),  # 20 / 12 scale bytes per row
    dict(T=200, n=40, k=6, d=512, latent=256, m=256, shared=320),    # ragged loads, column tails
    dict(T=16, n=64, k=4, d=256, latent=128, m=128, shared=128),     # decode-like: 1 row per expert
])
def test_w4a8_layer(kw):
    check_layer(workloads.small_shape(routed="mxfp4_a8", **kw), seed=11, name=f"w4a8 {kw}")


# W4A4: MXFP4 weights times MXFP4 activations on the scaled MFMA (320-row
# tiles only, E2M1 on both operands), against the oracle that rounds z and h
# to bf16 and then MXFP4
@pytest.mark.parametrize("kw", [
    dict(T=300, n=16, k=4, d=1024, latent=512, m=512, shared=256),   # 75 rows per expert
    dict(T=1200, n=16, k=4, d=1024, latent=512, m=512, shared=256),  # 300 rows per expert
    dict(T=1000, n=16, k=4, d=1024, latent=640, m=384, shared=256),  # 20 / 12 scale bytes per row
    dict(T=200, n=40, k=6, d=512, latent=256, m=256, shared=320),    # ragged loads, column tails
    dict(T=16, n=64, k=4, d=256, latent=128, m=128, shared=128),     # decode-like: 1 row per expert
])
def test_w4a4_layer(kw):
    check_layer(workloads.small_shape(routed="mxfp4_a4", **kw), seed=13, name=f"w4a4 {kw}")


def test_w4a4_layer_frozen_uneven_tiles():
    shape = workloads.small_shape(routed="mxfp4_a4", T=1000, n=16, k=4, d=1024, latent=512, m=512,
                                  shared=256, offset_std=1.0)
    check_layer(shape, seed=14, qb_mode=qb.MODE_FROZEN, bias=np.zeros(shape.n),
                name="w4a4 frozen, uneven 320-row tiles")


def test_w4a4_layer_extreme_scale_bytes():
    shape = workloads.small_shape(routed="mxfp4_a4", T=300, n=16, k=4, d=1024, latent=512,
                                  m=512, shared=256)
    check_layer(shape, seed=4, name="w4a4 extreme scales", edit=extreme_scale_bytes)


def test_w4a8_layer_empty_batch():
    import sparse_moe_ffn_sigmoid_amd as moe
    shape = workloads.small_shape(routed="mxfp4_a8", T=0, latent=128, m=128)
    inp = workloads.layer_inputs(shape, "cpu", seed=0)
    announce("w4a8 layer T=0")
    got = run_gpu(moe, shape, inp)
    assert got["out"].shape == (0, shape.d) and (got["loads"] == 0).all()


def test_w4a8_layer_frozen_uneven_tiles():
    shape = workloads.small_shape(routed="mxfp4_a8", T=1000, n=16, k=4, d=1024, latent=512, m=512,
                                  shared=256, offset_std=1.0)
    check_layer(shape, seed=12, qb_mode=qb.MODE_FROZEN, bias=np.zeros(shape.n),
                name="w4a8 frozen, uneven 320-row tiles")


def test_mxfp4_layer_frozen_zero_bias():
    shape = workloads.small_shape(routed="mxfp4", T=300, k=4, offset_std=1.0)
    check_layer(shape, seed=3, qb_mode=qb.MODE_FROZEN, bias=np.zeros(shape.n),
                name="mxfp4 frozen")


def test_bf16_layer_frozen_bias():
    shape = workloads.small_shape(T=120)
    bias = np.rint(np.random.default_rng(4).normal(0, 0.1, shape.n) * 2.0 ** 40) * 2.0 ** -40
    check_layer(shape, seed=4, qb_mode=qb.MODE_FROZEN, bias=bias, name="bf16 frozen")


def test_mxfp4_layer_frozen_uneven_320_row_tiles():
    # skewed router, frozen zero bias: loads from tens to several hundred
    # rows per expert on 320-row MXFP4 tiles (up to three tiles per expert)
    shape = workloads.small_shape(routed="mxfp4", T=1000, n=16, k=4, d=1024, latent=512, m=512,
                                  shared=256, offset_std=1.0)
    check_layer(shape, seed=9, qb_mode=qb.MODE_FROZEN, bias=np.zeros(shape.n),
                name="mxfp4 frozen, uneven 320-row tiles")


@pytest.mark.parametrize("seed", [8, 9])
def test_bf16_layer_frozen_uneven_tall_tiles(seed):
    # a skewed router with a frozen zero bias: 250 rows per expert on average
    # (320-row tiles), loads from 28 to 838 rows (up to three tiles, ragged)
    shape = workloads.small_shape(T=1000, n=16, k=4, offset_std=1.0)
    check_layer(shape, seed=seed, qb_mode=qb.MODE_FROZEN, bias=np.zeros(shape.n),
                name="bf16 frozen, uneven 320-row tiles")


def test_layer_empty_batch():
    import sparse_moe_ffn_sigmoid_amd as moe
    shape = workloads.small_shape(T=0)
    inp = workloads.layer_inputs(shape, "cpu", seed=0)
    announce("layer T=0")
    got = run_gpu(moe, shape, inp)
    assert got["out"].shape == (0, shape.d) and (got["loads"] == 0).all()


def test_bf16_decode_with_bias_from_a_qb_batch():
    # inference routing: QB balances a prefill batch, then a decode batch of
    # the same layer is routed with that bias frozen
    import sparse_moe_ffn_sigmoid_amd as moe
    pre = workloads.small_shape(T=400, k=4)
    inp = workloads.layer_inputs(pre, "cpu", seed=6, random_gamma=True)
    announce("prefill batch with QB")
    got_pre = run_gpu(moe, pre, inp)
    assert int(got_pre["info"][1]) == qb.STATUS_OK
    assert (got_pre["loads"] == qb.targets(pre.T, pre.n, pre.k)).all()
    dec = workloads.small_shape(T=16, k=4)
    check_layer(dec, seed=6, qb_mode=qb.MODE_FROZEN, bias=got_pre["bias"],
                name="decode, bias carried over")
