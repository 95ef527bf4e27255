"""Pins of the gradient oracle (oracle/grad.py).

* Its forward pass is the layer oracle's (an independent NumPy version).
* Every gradient, at sampled entries of every tensor, equals a central
  finite difference of sum(out * dout) computed with the NumPy layer oracle,
  the mixture weights recomputed from the float64 router scores and the
  selection held fixed (a dropped term, a wrong sign or a transposed
  operand in the autograd graph changes some entry by far more than the
  difference error).
* Closed forms: the gradient of the RMSNorm gain is sum_t (dout W_up)_t
  times the normalised routed row; experts and router rows that no token
  chose receive nothing.
"""
import numpy as np
import pytest

import workloads
from oracle import grad as ograd
from oracle import layer as olayer
from oracle import qb


def tiny(seed=0, T=6, offset=True):
    shape = workloads.small_shape(T=T, d=64, latent=32, n=6, k=2, m=16, shared=16, act="f32",
                                  routed="f32", offset_std=0.5 if offset else 0.0)
    inp = workloads.layer_inputs(shape, "cpu", seed=seed, random_gamma=True)
    inp = {k: (None if v is None else olayer.as_f64(v)) for k, v in inp.items()}
    s = olayer.router_scores(inp["x"], inp["w_router"], inp["logit_offset"])
    r = qb.route_qb(s, shape.k)
    dout = np.random.default_rng(seed + 100).standard_normal((T, shape.d))
    return shape, inp, r["idx"], dout


def objective(inp, idx, eps, dout):
    """sum(out * dout) with w recomputed from the float64 router scores."""
    logits = inp["x"] @ inp["w_router"].T
    if inp.get("logit_offset") is not None:
        logits = logits + inp["logit_offset"][None, :]
    s = olayer.sigmoid(logits)
    sel = np.take_along_axis(s, np.asarray(idx, np.int64), axis=1)
    w = sel / sel.sum(axis=1, keepdims=True)
    return float(np.sum(olayer.layer_forward(inp, idx, w, eps) * dout))


def test_forward_matches_layer_oracle():
    shape, inp, idx, dout = tiny()
    g = ograd.layer_grads(inp, idx, shape.eps, dout)
    s = olayer.sigmoid(inp["x"] @ inp["w_router"].T + inp["logit_offset"][None, :])
    sel = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    ref = olayer.layer_forward(inp, idx, sel / sel.sum(1, keepdims=True), shape.eps)
    assert np.allclose(g["out"], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("key", list(ograd.GRAD_KEYS))
def test_gradients_match_finite_differences(key):
    shape, inp, idx, dout = tiny(seed=3)
    g = ograd.layer_grads(inp, idx, shape.eps, dout)[key]
    rng = np.random.default_rng(7)
    flat = inp[key].reshape(-1)
    picks = rng.choice(flat.size, size=min(12, flat.size), replace=False)
    if key in ("w_gate", "w_uproj", "w_dn"):          # entries of experts that were chosen
        used = np.unique(idx)
        per = flat.size // shape.n
        picks = np.array([int(rng.choice(used)) * per + int(rng.integers(per)) for _ in range(12)])
    for i in picks:
        h = 1e-6 * max(1.0, abs(flat[i]))
        old = flat[i]
        flat[i] = old + h
        fp = objective(inp, idx, shape.eps, dout)
        flat[i] = old - h
        fm = objective(inp, idx, shape.eps, dout)
        flat[i] = old
        fd = (fp - fm) / (2 * h)
        an = g.reshape(-1)[i]
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (key, i, fd, an)


def test_unchosen_experts_get_no_gradient():
    shape, inp, idx, dout = tiny(seed=4)
    g = ograd.layer_grads(inp, idx, shape.eps, dout)
    unused = np.setdiff1d(np.arange(shape.n), np.unique(idx))
    for key in ("w_gate", "w_uproj", "w_dn"):
        assert (g[key][unused] == 0).all()
    # router rows of experts never chosen get none either (w only sees the chosen scores)
    assert (g["w_router"][unused] == 0).all() and (g["logit_offset"][unused] == 0).all()


def test_rms_gain_gradient_closed_form():
    shape, inp, idx, dout = tiny(seed=5)
    g = ograd.layer_grads(inp, idx, shape.eps, dout)
    # d/dgamma of sum(dout * (yn W_up^T)) = sum_t (dout W_up)_t * y_t r_t
    s = olayer.sigmoid(inp["x"] @ inp["w_router"].T + inp["logit_offset"][None, :])
    sel = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    w = sel / sel.sum(1, keepdims=True)
    z = inp["x"] @ inp["w_down"].T
    y = np.zeros((inp["x"].shape[0], z.shape[1]))
    for t in range(y.shape[0]):
        for j, e in enumerate(idx[t]):
            h = olayer.situ_glu(z[t] @ inp["w_gate"][e].T, z[t] @ inp["w_uproj"][e].T)
            y[t] += w[t, j] * (h @ inp["w_dn"][e].T)
    yr = y / np.sqrt(np.mean(y * y, axis=1, keepdims=True) + shape.eps)
    want = np.sum((dout @ inp["w_up"]) * yr, axis=0)
    assert np.allclose(g["rms_gamma"], want, rtol=1e-10, atol=1e-12)


def _round_rne(x, mant_bits):
    """Exact rational x rounded to the nearest binary float with `mant_bits`
    significant bits (ties to even); normal range only."""
    from fractions import Fraction
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(Fraction(x))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (e - mant_bits + 1)
    q, r = divmod(a, ulp)
    q = int(q)
    if r * 2 > ulp or (r * 2 == ulp and q % 2 == 1):
        q += 1
    return sign * q * ulp


def test_sgd_step_hand_cases():
    # exact: 1.5 - 1 * 0.25; ties to even at the bf16 grid of [1, 2) (spacing 2^-7)
    w = np.array([1.5, 1 + 2 ** -7, 1 + 2 ** -6])
    g = np.array([0.25, 2 ** -8, 2 ** -8])
    assert ograd.sgd_step(w, g, 1.0, "bf16").tolist() == [1.25, 1.0, 1.015625]
    # fp32 weights keep 1 + 2^-8
    assert ograd.sgd_step(w, g, 1.0, "f32").tolist() == [1.25, 1 + 2 ** -8, 1 + 3 * 2 ** -8]


def test_sgd_step_matches_exact_rounding():
    """Against the definition in exact rational arithmetic: the product and
    the difference each rounded to 24 bits, then (bf16) to 8 bits.  Some
    samples would come out differently with a single rounding of w - lr*g
    (a fused multiply-add), so that mistake fails here."""
    from fractions import Fraction
    rng = np.random.default_rng(3)
    w = (rng.standard_normal(400) * 0.05).astype(np.float32)
    g = (rng.standard_normal(400) * 3.0).astype(np.float32)
    lr = np.float32(0.0123)
    fused_differs = 0
    for dtype, bits in (("f32", 24), ("bf16", 8)):
        wd = w if dtype == "f32" else ograd.layer.bf16_round(w.astype(np.float64)).astype(np.float32)
        got = ograd.sgd_step(wd, g, float(lr), dtype)
        for i in range(w.size):
            t = _round_rne(Fraction(float(lr)) * Fraction(float(g[i])), 24)
            r = _round_rne(Fraction(float(wd[i])) - t, 24)
            want = _round_rne(r, bits) if bits < 24 else r
            assert Fraction(float(got[i])) == want, (dtype, i)
            fused = _round_rne(Fraction(float(wd[i])) - Fraction(float(lr)) * Fraction(float(g[i])), 24)
            fused_differs += int((_round_rne(fused, bits) if bits < 24 else fused) != want)
    assert fused_differs > 0
