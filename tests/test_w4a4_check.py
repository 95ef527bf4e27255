"""The W4A4 test helper in layer_cases (per-token recomputation with one
bf16 rounding taken the other way) against the oracle layer."""
import numpy as np

import workloads
from layer_cases import _ambiguous, _w4a4_token, oracle_scores
from oracle import layer as olayer
from oracle import qb


def test_token_helper_is_the_oracle_layer():
    shape = workloads.small_shape(routed="mxfp4_a4", T=24, n=16, k=4, d=256, latent=128, m=128,
                                  shared=128)
    inp = workloads.layer_inputs(shape, "cpu", seed=6, random_gamma=True)
    r = qb.route_qb(oracle_scores(inp), shape.k)
    ref = olayer.layer_forward(inp, r["idx"], r["w"], shape.eps, act_mxfp4=True)
    for t in (0, 7, 23):
        out, _, _ = _w4a4_token(inp, t, r["idx"][t], r["w"][t], shape.eps)
        assert np.allclose(out, ref[t], rtol=1e-12, atol=1e-12)


def test_ambiguous_roundings():
    # 1 + 2^-8 is a bf16 midpoint (between 1 and 1 + 2^-7); 1 + 2^-9 is not
    v = np.array([1.0 + 2.0 ** -8, 1.0 + 2.0 ** -9, -(3.0 + 3 * 2.0 ** -7)])
    idx, other = _ambiguous(v)
    assert idx.tolist() == [0, 2]
    assert other[0] == 1.0 + 2.0 ** -7          # RNE takes 1; the other neighbour
    assert other[1] in (-3.0 - 2.0 ** -6, -3.0 - 2 * 2.0 ** -6)
