"""Pins of the layer oracle: closed forms, bounds and identities the pages fix."""
import numpy as np
import pytest
import torch

import perm_layer
import workloads
from oracle import layer, qb


def test_sigmoid_closed_forms():
    assert layer.sigmoid(0.0) == 0.5
    assert abs(layer.sigmoid(np.log(3.0)) - 0.75) < 1e-15


def test_situ_glu_closed_form_point():
    # gate 4*atanh(1/2) caps to 2, up 25*atanh(1/2) caps to 12.5:
    # h = SiLU(2) * 12.5 = 2*sigmoid(2)*12.5 (a swap of beta1/beta2 fails this)
    g = 4 * np.arctanh(0.5)
    u = 25 * np.arctanh(0.5)
    want = 2.0 / (1.0 + np.exp(-2.0)) * 12.5
    assert abs(layer.situ_glu(g, u) - want) < 1e-12


def test_situ_glu_bound_and_symmetries():
    v = np.sort(np.concatenate([np.linspace(-50, 50, 2001), [-1e4, -1e3, 1e3, 1e4]]))
    G, U = np.meshgrid(v, v)          # G varies along columns, U along rows
    h = layer.situ_glu(G, U)
    sup = 25 * 4 / (1 + np.exp(-4.0))           # 98.2014...: bounded by 100
    assert np.abs(h).max() <= sup + 1e-12 and sup < 100
    assert np.abs(h).max() > 98.0
    assert (layer.situ_glu(0.0, v) == 0).all() and (layer.situ_glu(v, 0.0) == 0).all()
    assert np.allclose(layer.situ_glu(G, -U), -h, atol=0)
    # monotone in u, with the sign of SiLU(capped gate)
    du = np.diff(h, axis=0)
    assert (du[:, v > 0] >= 0).all() and (du[:, v < 0] <= 0).all()


def test_situ_glu_matches_swiglu_near_origin():
    rng = np.random.default_rng(0)
    g = rng.uniform(-0.01, 0.01, 1000)
    u = rng.uniform(-0.01, 0.01, 1000)
    swiglu = g / (1 + np.exp(-g)) * u
    rel = np.abs(layer.situ_glu(g, u) - swiglu) / np.abs(swiglu)
    assert rel.max() < 1e-5


def test_rmsnorm_closed_form_and_scale_invariance():
    y = np.array([[3.0, 4.0]])
    out = layer.rmsnorm(y, np.ones(2), 0.0)
    assert np.allclose(out, y / np.sqrt(12.5), rtol=1e-15)
    rng = np.random.default_rng(1)
    y = rng.standard_normal((8, 64))
    g = rng.uniform(0.5, 1.5, 64)
    o = layer.rmsnorm(y, g, 1e-6)
    assert np.allclose(np.sqrt(np.mean((o / g) ** 2, axis=1)), 1.0, atol=1e-5)
    assert np.allclose(layer.rmsnorm(7.5 * y, g, 1e-6), o, atol=1e-7)


def test_mxfp4_code_table_and_nibble_order():
    codes = np.array([[0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE] * 2], np.uint8)
    v = layer.mxfp4_decode(codes, np.array([[127]], np.uint8))[0]
    mags = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(v[:16]) == mags + [-m for m in mags]
    v8 = layer.mxfp4_decode(codes, np.array([[130]], np.uint8))[0]
    assert (v8 == 8 * v).all()


def test_mxfp4_quantiser_round_trip():
    rng = np.random.default_rng(0)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    vals = rng.choice(mags, size=(6, 64)) * rng.choice([-1, 1], size=(6, 64))
    vals[:, 0] = 6.0                               # amax 6 per block -> exponent 0
    vals[:, 32] = -6.0
    for E in (-7, 0, 3):
        w = torch.tensor(vals * 2.0 ** E, dtype=torch.float32)
        codes, scales = workloads.mxfp4_quantize(w)
        assert (scales.numpy() == 127 + E).all()
        back = layer.mxfp4_decode(codes.numpy(), scales.numpy())
        assert (back == vals * 2.0 ** E).all()
    # rounding: ties to the even code, saturation at 6
    w = torch.tensor([[0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.9] + [6.0] + [0.0] * 23])
    codes, scales = workloads.mxfp4_quantize(w)
    back = layer.mxfp4_decode(codes.numpy(), scales.numpy())[0]
    assert list(back[:9]) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0]


def test_shared_experts_merge_is_sum_of_two():
    rng = np.random.default_rng(3)
    d, m = 32, 12
    x = rng.standard_normal((5, d))
    wg, wu, wd = rng.standard_normal((m, d)), rng.standard_normal((m, d)), rng.standard_normal((d, m))
    merged = layer.shared_mlp(x, wg, wu, wd)
    h = m // 2
    two = (layer.shared_mlp(x, wg[:h], wu[:h], wd[:, :h]) +
           layer.shared_mlp(x, wg[h:], wu[h:], wd[:, h:]))
    assert np.allclose(merged, two, rtol=1e-12, atol=1e-12)


def _tiny_inputs(**kw):
    shape = workloads.small_shape(T=48, d=64, latent=32, n=8, k=2, m=16, shared=24,
                                  act="f32", routed="f32", **kw)
    return shape, workloads.layer_inputs(shape, "cpu", seed=1, random_gamma=True)


def test_layer_rmsnorm_placement_after_aggregation():
    # scaling every routed down-projection by c > 0 (a power of two, so the
    # fp32 weights scale exactly) scales the aggregated
    # latent sum by c; RMSNorm before the up-projection removes it.
    shape, inp = _tiny_inputs()
    r = layer.route_layer(inp, shape.k)
    out = layer.layer_forward(inp, r["idx"], r["w"], 0.0)
    inp2 = dict(inp)
    inp2["w_dn"] = inp["w_dn"] * 4.0          # exact in fp32
    out2 = layer.layer_forward(inp2, r["idx"], r["w"], 0.0)
    assert np.allclose(out, out2, rtol=1e-10, atol=1e-10)
    # ... whereas scaling the latent projection does change the output
    inp3 = dict(inp)
    inp3["w_down"] = inp["w_down"] * 3.0
    out3 = layer.layer_forward(inp3, r["idx"], r["w"], 0.0)
    assert not np.allclose(out, out3, rtol=1e-3, atol=1e-3)


def test_layer_without_routed_signal_is_shared_mlp():
    shape, inp = _tiny_inputs()
    r = layer.route_layer(inp, shape.k)
    inp2 = dict(inp)
    inp2["w_dn"] = torch.zeros_like(inp["w_dn"])
    out = layer.layer_forward(inp2, r["idx"], r["w"], shape.eps)
    ref = layer.shared_mlp(inp["x"], inp["ws_gate"], inp["ws_up"], inp["ws_down"])
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_layer_token_sampling_matches_full():
    shape, inp = _tiny_inputs()
    r = layer.route_layer(inp, shape.k)
    assert r["info"][1] == qb.STATUS_OK
    full = layer.layer_forward(inp, r["idx"], r["w"], shape.eps)
    some = layer.layer_forward(inp, r["idx"], r["w"], shape.eps, tokens=[3, 17, 40])
    assert np.allclose(full[[3, 17, 40]], some, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("act_fmt,mx", [(None, False), ("mxfp8", False), (None, True),
                                        ("mxfp8", True), ("mxfp4", True)])
def test_layer_composition_with_permutation_weights(act_fmt, mx):
    """The whole layer on scaled permutation weights against its output
    written out by hand (``tests/perm_layer.py``).  With ``act_fmt`` the
    expert inputs z and the SiTU-GLU outputs h (rows of 64, two blocks) are
    rounded to bf16 and then MXFP8 (W4A8) or MXFP4 (W4A4) at exactly those
    two places, with the separately pinned codecs.  With ``mx`` the routed
    experts are given as MXFP4 codes and E8M0 scales whose values E2M1 x 2^E
    holds exactly."""
    inp, par = perm_layer.build(exact_mxfp4=mx)
    if mx:
        for key in ("w_gate", "w_uproj", "w_dn"):
            codes, scales = workloads.mxfp4_quantize(torch.from_numpy(inp[key].reshape(-1, perm_layer.LAT)))
            n, lat = perm_layer.N, perm_layer.LAT
            inp[key] = (codes.reshape(n, lat, lat // 2), scales.reshape(n, lat, lat // 32))
    r = layer.route_layer(inp, perm_layer.K, mode=qb.MODE_FROZEN, bias=np.zeros(perm_layer.N))
    assert (r["idx"] == perm_layer.TOP).all()
    sc = 1.0 / (1.0 + np.exp(-perm_layer.LOGIT_OFFSET))
    top = sc[perm_layer.TOP]
    assert np.allclose(r["w"], (top / top.sum())[None, :], rtol=1e-6, atol=0)
    out = layer.layer_forward(inp, r["idx"], r["w"], perm_layer.EPS,
                              act_mxfp8=act_fmt == "mxfp8", act_mxfp4=act_fmt == "mxfp4")
    fn = {"mxfp8": layer.w4a8_activation, "mxfp4": layer.w4a4_activation}.get(act_fmt)
    act = (lambda v: fn(v[None, :])[0]) if fn else (lambda v: v)
    want = perm_layer.expected(inp, par, r["idx"], r["w"], act)
    assert np.allclose(out, want, rtol=1e-12, atol=1e-12)


def test_router_scores_with_zero_input_are_sigmoid_of_offset():
    p = np.array([-1.0, 0.0, 2.0])
    s = layer.router_scores(np.zeros((2, 4)), np.ones((3, 4)), p)
    assert s.dtype == np.float32
    assert np.allclose(s, 1 / (1 + np.exp(-p))[None, :], rtol=1e-7)


# --- MXFP8 (E4M3) activations of the W4A8 experts: OCP Microscaling v1.0 ---

def test_e4m3_code_table():
    c = np.arange(256, dtype=np.uint8)
    v = layer.e4m3_decode(c)
    # the format's landmarks: smallest subnormal 2^-9, smallest normal 2^-6,
    # one (0x38), largest finite 448 = 1.75 * 2^8, NaN at S.1111.111 only
    assert v[0x00] == 0 and v[0x01] == 2.0 ** -9 and v[0x07] == 7 * 2.0 ** -9
    assert v[0x08] == 2.0 ** -6 and v[0x38] == 1.0 and v[0x39] == 1.125 and v[0x3C] == 1.5
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0
    assert np.isnan(v[[0x7F, 0xFF]]).all() and np.isnan(v).sum() == 2
    assert (np.diff(v[:0x7F]) > 0).all()                     # positive codes increase
    assert (v[0x80:0xFF] == -v[:0x7F]).all()                 # the sign bit only negates
    fin = ~np.isnan(v)
    assert (layer.e4m3_encode(v[fin]) == c[fin]).all()       # every finite value round-trips


def test_e4m3_rounding_ties_and_saturation():
    enc = layer.e4m3_encode
    # ties between neighbours go to the even mantissa
    assert enc(np.array([1.0625]))[0] == 0x38 and enc(np.array([1.1875]))[0] == 0x3A
    assert enc(np.array([2.0 ** -10]))[0] == 0x00 and enc(np.array([3 * 2.0 ** -10]))[0] == 0x02
    # just off a tie rounds to the nearer value
    assert enc(np.array([1.0625 + 1e-9]))[0] == 0x39
    # saturation at 448 instead of overflow to NaN
    assert (layer.e4m3_decode(enc(np.array([449.0, 464.0, 1e6, -1e6]))) == [448, 448, 448, -448]).all()
    # brute force: the encoded value is a nearest finite E4M3 value
    grid = layer.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    x = np.random.default_rng(0).uniform(0, 448, 20000) * 2.0 ** np.random.default_rng(1).integers(-14, 1, 20000)
    r = layer.e4m3_decode(enc(x))
    best = np.abs(grid[None, :] - x[:, None]).min(axis=1)
    assert np.array_equal(np.abs(r - x), best)


def test_mxfp8_block_scale_rule_and_error_bound():
    rng = np.random.default_rng(2)
    v = rng.normal(0, 1, (64, 256)) * np.exp(rng.normal(0, 3, (64, 1)))
    v[3, 32:64] = 0.0                                       # an all-zero block
    codes, sb = layer.mxfp8_quantize(v)
    assert codes.shape == v.shape and sb.shape == (64, 8)
    amax = np.abs(v.reshape(64, 8, 32)).max(axis=2)
    nz = amax > 0
    # shared exponent floor(log2 amax) - 8: the block maximum lands in [2^8, 2^9)
    X = sb.astype(np.int64) - 127
    assert ((amax[nz] >= 2.0 ** (X[nz] + 8)) & (amax[nz] < 2.0 ** (X[nz] + 9))).all()
    assert sb[3, 1] == 0 and (codes[3, 32:64] == 0).all()
    d = layer.mxfp8_decode(codes, sb)
    # error bound: half a unit in the last place, relative 2^-4 for normals, and
    # the saturation of block maxima in (448, 512) * 2^X
    ulp = np.maximum(np.abs(v), np.repeat(2.0 ** (X + 2), 32, axis=1))
    sat = np.abs(v) > 448 * np.repeat(2.0 ** X, 32, axis=1)
    assert (np.abs(d - v)[~sat] <= ulp[~sat] * 2.0 ** -4 + 1e-300).all()
    assert (np.abs(d[sat]) == 448 * np.repeat(2.0 ** X, 32, axis=1)[sat]).all()
    # exactly representable blocks come back unchanged
    grid = layer.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    w = rng.choice(grid[grid > 0], (8, 64)) * 2.0 ** -5
    w[:, ::32] = 256 * 2.0 ** -5                              # block maximum 2^8 * 2^X
    assert np.array_equal(layer.mxfp8_round(w), w)


# --- MXFP4 (E2M1) activations, the oracle side of a W4A4 reading ---------

def test_e2m1_ties_and_saturation():
    # midpoints of neighbouring E2M1 values go to the one with a zero
    # mantissa bit (0, 1, 2, 4 are even, 0.5, 1.5, 3, 6 odd); above 6 saturates
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, 1e9])
    want = np.array([0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0])
    for sign in (1.0, -1.0):
        c = layer.e2m1_encode(sign * mids)
        got = layer.E2M1_VALUES[c & 7] * np.where(c & 8, -1.0, 1.0)
        assert (got == sign * want).all()
        assert ((c & 8) != 0).all() == (sign < 0)


def test_mxfp4_act_nearest_value_and_block_rule():
    rng = np.random.default_rng(5)
    v = rng.normal(0, 1, (64, 64)) * np.exp2(rng.integers(-20, 20, (64, 1)))
    r = layer.mxfp4_act_round(v)
    blk, rb = v.reshape(64, 2, 32), r.reshape(64, 2, 32)
    amax = np.abs(blk).max(axis=2)
    X = np.floor(np.log2(amax)) - 2                       # 6 * 2^X >= amax > 2^(X+2)
    grid = layer.E2M1_VALUES[None, None, :] * np.exp2(X)[:, :, None]
    nearest = np.abs(np.abs(blk)[..., None] - grid[:, :, None, :]).min(axis=-1)
    # every result is a grid value, and no grid value is nearer (brute force)
    assert (np.abs(np.abs(rb)[..., None] - grid[:, :, None, :]).min(axis=-1) == 0).all()
    assert np.array_equal(np.abs(np.abs(blk) - np.abs(rb)), nearest)
    assert (np.sign(rb) * np.sign(blk) >= 0).all()
    # representable values round-trip exactly
    exact = layer.E2M1_VALUES[rng.integers(0, 8, (4, 32))] * np.where(rng.random((4, 32)) < .5, -1, 1)
    exact[:, 0] = 6.0                                      # fixes the block scale at 2^0
    assert (layer.mxfp4_act_round(exact * 2.0 ** -7) == exact * 2.0 ** -7).all()


def test_mxfp4_act_matches_the_weight_quantiser():
    # two independent implementations of the same OCP rule (the seeded weight
    # generator's quantiser in torch float32, the oracle's in float64)
    rng = np.random.default_rng(9)
    v = (rng.normal(0, 1, (16, 128)) * np.exp2(rng.integers(-8, 8, (16, 1)))).astype(np.float32)
    codes, scales = workloads.mxfp4_quantize(torch.from_numpy(v))
    assert np.array_equal(layer.mxfp4_decode(codes.numpy(), scales.numpy()),
                          layer.mxfp4_act_round(v.astype(np.float64)))


def test_w4a4_activation_rounds_bf16_first():
    # 1.25 + 2^-12 is 1.25 in bf16; in a block with amax ~1.25 (scale 2^-2)
    # that is 5 units, the midpoint of 4 and 6, which goes to 4 (1.0); the
    # float64 value rounds up to 6 units (1.5) instead.
    v = np.zeros((1, 32))
    v[0, 0] = 1.25 + 2.0 ** -12
    assert layer.mxfp4_act_round(v)[0, 0] == 1.5
    assert layer.w4a4_activation(v)[0, 0] == 1.0


def test_w4a8_activation_rounds_bf16_first():
    # The expert reads its bf16-stored input: 1.0625 + 2^-12 becomes 1.0625
    # in bf16, which sits exactly between the E4M3 neighbours 1 and 1.125 of
    # its block (amax ~1.06: scale 2^-8) and goes to the even one, 1.  A
    # direct MXFP8 rounding of the float64 value gives 1.125 instead.
    v = np.zeros((1, 32))
    v[0, 0] = 1.0625 + 2.0 ** -12
    assert layer.bf16_round(v)[0, 0] == 1.0625
    assert layer.mxfp8_round(v)[0, 0] == 1.125
    assert layer.w4a8_activation(v)[0, 0] == 1.0


def test_w4a8_layer_moves_by_the_activation_rounding():
    shape = workloads.small_shape(routed="mxfp4", T=48, k=4, n=16, d=256, latent=128, m=128,
                                  shared=128)
    inp = workloads.layer_inputs(shape, "cpu", seed=4)
    s = layer.router_scores(layer.as_f64(inp["x"]), layer.as_f64(inp["w_router"]),
                            layer.as_f64(inp["logit_offset"]))
    r = qb.route_qb(s, shape.k)
    a16 = layer.layer_forward(inp, r["idx"], r["w"], shape.eps)
    a8 = layer.layer_forward(inp, r["idx"], r["w"], shape.eps, act_mxfp8=True)
    # E4M3 rounding (ties to even) leaves a relative error uniform within
    # +-2^-4 of each element of z and h: rms 2^-4 / sqrt(3) = 3.6% each.  The
    # routed half of the output moves by about that much; rms(a8 - a16) / rms(a16)
    # must lie well inside (0.5%, 8%)
    rel_rms = np.sqrt(np.mean((a8 - a16) ** 2) / np.mean(a16 ** 2))
    assert 0.005 < rel_rms < 0.08
    # no rounding at all when the activations already sit on the MXFP8 grid
    z = layer.as_f64(inp["x"]) @ layer.as_f64(inp["w_down"]).T
    q = layer.w4a8_activation(z)
    assert np.array_equal(layer.w4a8_activation(q), q)


def test_w4a4_layer_moves_by_the_activation_rounding():
    shape = workloads.small_shape(routed="mxfp4", T=48, k=4, n=16, d=256, latent=128, m=128,
                                  shared=128)
    inp = workloads.layer_inputs(shape, "cpu", seed=4)
    s = layer.router_scores(layer.as_f64(inp["x"]), layer.as_f64(inp["w_router"]),
                            layer.as_f64(inp["logit_offset"]))
    r = qb.route_qb(s, shape.k)
    a16 = layer.layer_forward(inp, r["idx"], r["w"], shape.eps)
    a8 = layer.layer_forward(inp, r["idx"], r["w"], shape.eps, act_mxfp8=True)
    a4 = layer.layer_forward(inp, r["idx"], r["w"], shape.eps, act_mxfp4=True)
    # E2M1 keeps one mantissa bit: relative rounding error up to 1/6 near the
    # top of a binade, rms around 8% of each element of z and h, and values
    # below 1/8 of the block maximum mostly rounded to 0 or 0.5.  The routed half
    # of the output moves by several times the W4A8 change, but well under 100%
    e4 = np.sqrt(np.mean((a4 - a16) ** 2) / np.mean(a16 ** 2))
    e8 = np.sqrt(np.mean((a8 - a16) ** 2) / np.mean(a16 ** 2))
    assert 2 * e8 < e4 < 0.5
    z = layer.as_f64(inp["x"]) @ layer.as_f64(inp["w_down"]).T
    q = layer.w4a4_activation(z)
    assert np.array_equal(layer.w4a4_activation(q), q)


def test_bf16_round_ties_to_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties to even (1)
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8)])
    assert np.array_equal(layer.bf16_round(v), [1.0, 1.0 + 2.0 ** -6, -1.0])
