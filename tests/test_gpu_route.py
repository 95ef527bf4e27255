"""Parity of moe_route_qb (HIP) with the QB oracle, through the C ABI.

Bit-exact on indices, loads, the returned bias and the round/move counts
(the HIP path runs the same schedule); weights within (k+1) fp32 ulps of
the float64 oracle.  Inputs: router logits N(0,1) plus a per-expert offset,
turned into fp32 scores by the oracle's sigmoid and fed to both sides.
"""
import json
import os
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle import layer as olayer
from oracle import qb

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def scores(T, n, offset_std=0.5, seed=0):
    return olayer.sigmoid(workloads.qb_logits(T, n, offset_std, seed)).astype(np.float32)


def gpu_route(s, k, bias=None, mode=1, max_rounds=64):
    import sparse_moe_ffn_sigmoid_amd as moe
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float64)).cuda()
    r = moe.route_qb(torch.from_numpy(s).cuda(), k, b, mode, max_rounds)
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in r.items()}


def announce(name):
    print(f"\n[gpu case] {name}", flush=True)
    sys.stdout.flush()


def check(s, k, mode=qb.MODE_BATCH, bias=None, name=""):
    announce(f"route {name} T={s.shape[0]} n={s.shape[1]} k={k} mode={mode}")
    ref = qb.route_qb(s, k, bias=bias, mode=mode)
    got = gpu_route(s, k, bias, mode)
    assert (got["idx"] == ref["idx"]).all()
    assert (got["loads"] == ref["loads"]).all()
    assert tuple(int(v) for v in got["info"]) == tuple(ref["info"])
    if mode == qb.MODE_BATCH:
        assert (got["bias"] == ref["bias"]).all()
    tol = (k + 1) * 2.0 ** -24
    assert np.allclose(got["w"], ref["w"], rtol=tol, atol=0)
    return ref, got


CASES = [
    ("tiny", 64, 32, 4, 0.3),
    ("decode", 64, 896, 16, 0.5),
    ("ragged", 1000, 100, 7, 1.0),
    ("mid", 3000, 256, 8, 0.5),
    ("max_n_k", 300, 1024, 64, 0.5),
    ("k3_prefill_shape", 4096, 896, 16, 0.5),
    # top-k pivots: lanes without keys (n < 64), k + 1 = n, k + 1 = 64,
    # several tokens per wave (T above three resident blocks per CU x 4)
    ("pivot_small_n", 500, 48, 20, 0.5),
    ("pivot_k_n_minus_1", 300, 40, 39, 0.5),
    ("pivot_k63", 400, 200, 63, 0.5),
    ("pivot_tokens_per_wave", 7000, 128, 6, 1.0),
    # quantile rounds of large batches: past the 2-byte bucket cache in LDS
    # (about 41 K tokens) each token keeps a 1-byte coarse bucket; past twice
    # that, the gather recomputes every margin
    ("coarse_bucket_cache", 60000, 16, 2, 0.5),
    ("uncached_gather", 120000, 16, 2, 0.5),
    # fewer tokens than the four waves of one top-k block; every target 0 or 1
    ("one_token", 1, 64, 4, 0.5),
    ("three_tokens", 3, 64, 4, 0.5),
    ("two_tokens_k3_width", 2, 896, 16, 0.5),
]


@pytest.mark.parametrize("name,T,n,k,std", CASES)
def test_route_batch_parity(name, T, n, k, std):
    ref, got = check(scores(T, n, std), k, name=name)
    assert ref["info"][1] == qb.STATUS_OK
    assert (got["loads"] == qb.targets(T, n, k)).all()


def clustered_scores(protos, copies, n, noise, seed):
    """`protos` random score rows, each repeated `copies` times with a
    distinct uniform perturbation of size `noise` per entry: the margins of
    an expert then form a few tight clusters of `copies` tokens each."""
    rng = np.random.default_rng(seed)
    base = olayer.sigmoid(rng.standard_normal((protos, n)))
    s = np.repeat(base, copies, axis=0) + noise * rng.random((protos * copies, n))
    return np.clip(s, 0.0, 1.0).astype(np.float32)


@pytest.mark.parametrize("protos,copies,n,k,seed", [(3, 4500, 6, 2, 1), (4, 5000, 8, 2, 2)])
def test_route_clustered_margins_parity(protos, copies, n, k, seed):
    """Thousands of distinct margins inside one relative width of a few
    percent around each unbalanced expert's target rank (every quantile
    round here has 6,000 - 10,000 of them in the buckets it must resolve,
    more than the 4,096 margins the quantile kernel ranks in LDS), so the
    rounds go through its exact radix selection over all tokens.  The
    balanced answer is still unique (no two margins are equal)."""
    s = clustered_scores(protos, copies, n, 1e-5, seed)
    ref, got = check(s, k, name=f"clustered {protos}x{copies}")
    assert ref["info"][1] == qb.STATUS_OK and ref["info"][0] > 0
    assert (got["loads"] == qb.targets(s.shape[0], n, k)).all()


@pytest.mark.parametrize("T,n,k,max_rounds", [(1000, 64, 4, 2), (600, 48, 3, 1), (2000, 128, 8, 3)])
def test_route_round_cap_hands_over_to_paths(T, n, k, max_rounds):
    """A small cap on the quantile rounds leaves tens of units of imbalance
    to the augmenting paths (53 - 81 moves here); the result and every
    counter must still match."""
    s = scores(T, n, 0.5)
    ref = qb.route_qb(s, k, max_rounds=max_rounds)
    announce(f"round cap {max_rounds} T={T} n={n} k={k}")
    got = gpu_route(s, k, max_rounds=max_rounds)
    assert ref["info"][0] == max_rounds and ref["info"][1] == qb.STATUS_OK and ref["info"][3] > 0
    assert tuple(int(v) for v in got["info"]) == tuple(ref["info"])
    assert (got["idx"] == ref["idx"]).all() and (got["bias"] == ref["bias"]).all()
    assert (got["loads"] == qb.targets(T, n, k)).all()


def test_route_frozen_parity():
    s = scores(500, 64, 1.0, seed=3)
    bias = np.random.default_rng(0).normal(0, 0.2, 64)
    bias = np.rint(bias * 2.0 ** 40) * 2.0 ** -40
    check(s, 6, mode=qb.MODE_FROZEN, bias=bias, name="frozen")


def test_route_warm_start_is_fixed_point():
    s = scores(2000, 128, 0.5, seed=5)
    ref = qb.route_qb(s, 8)
    announce("warm start")
    got = gpu_route(s, 8, bias=ref["bias"])
    assert tuple(int(v) for v in got["info"]) == (0, 0, 0, 0)
    assert (got["bias"] == ref["bias"]).all() and (got["idx"] == ref["idx"]).all()


def test_route_edge_cases():
    check(scores(50, 1, 0.5), 1, name="n=1")
    check(scores(20, 8, 0.5), 8, name="k=n")
    announce("T=0")
    got = gpu_route(np.zeros((0, 16), np.float32), 3)
    assert got["idx"].shape == (0, 3) and (got["loads"] == 0).all() and got["info"][1] == 0


def test_route_degenerate_reports_not_balanced():
    s = np.tile(np.array([[0.7, 0.3]], np.float32), (4, 1))
    announce("degenerate")
    got = gpu_route(s, 1, max_rounds=8)
    assert got["info"][1] == qb.STATUS_NOT_BALANCED
    ref = qb.route_qb(s, 1, max_rounds=8, max_sap=8)
    assert ref["info"][1] == qb.STATUS_NOT_BALANCED


def test_route_bias_out_of_range_reported():
    s = scores(100, 16, 0.5)
    announce("bias range")
    got = gpu_route(s, 2, bias=np.full(16, 2048.0), mode=qb.MODE_FROZEN)
    assert got["info"][1] == qb.STATUS_BIAS_RANGE


def test_route_qb_workload_full_size():
    """T=57344, n=896, k=16: against the stored oracle result, plus the
    optimality certificate (exact loads and a bias that reproduces the
    selection) checked here with plain NumPy."""
    path = os.path.join(GOLDEN, "qb_57344x896_k16.json")
    cfg = workloads.QB_SHAPE
    s = scores(cfg["T"], cfg["n"], cfg["offset_std"], seed=0)
    announce("qb full size")
    got = gpu_route(s, cfg["k"])
    C = qb.targets(cfg["T"], cfg["n"], cfg["k"])
    assert (got["loads"] == C).all() and got["info"][1] == 0
    # certificate: top-k of fixed-point (score + returned bias) is the selection
    sfx = np.rint(s.astype(np.float64) * 2.0 ** 40).astype(np.int64)
    bfx = np.rint(got["bias"] * 2.0 ** 40).astype(np.int64)
    key = ((sfx + bfx[None, :] + (1 << 51)) << 10) | (1023 - np.arange(cfg["n"]))
    top = np.argpartition(-key, cfg["k"] - 1, axis=1)[:, :cfg["k"]]
    assert (np.sort(top, 1) == np.sort(got["idx"], 1)).all()
    if os.path.exists(path):
        gold = json.load(open(path))
        import hashlib
        assert hashlib.sha256(got["idx"].astype("<i4").tobytes()).hexdigest() == gold["idx_sha256"]
        assert [int(v) for v in np.rint(got["bias"] * 2.0 ** 40)] == gold["bias_fixed"]
        assert [int(v) for v in got["info"]] == gold["info"]


# --- the fixed-step sign update baseline ----------------------------------

def gpu_sign(s, k, step, rounds, bias=None):
    import sparse_moe_ffn_sigmoid_amd as moe
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float64)).cuda()
    r = moe.route_sign(torch.from_numpy(s).cuda(), k, step, rounds, b)
    torch.cuda.synchronize()
    return {key: v.cpu().numpy() for key, v in r.items()}


SIGN_CASES = [
    ("tiny", 64, 32, 4, 0.3, 2.0 ** -12, 300),
    ("decode", 64, 896, 16, 0.5, 2.0 ** -10, 64),
    ("ragged", 1000, 100, 7, 1.0, 2.0 ** -9, 100),
    ("k3_prefill_shape", 4096, 896, 16, 0.5, 2.0 ** -10, 64),
    ("no_rounds", 500, 64, 8, 0.5, 2.0 ** -10, 0),
]


@pytest.mark.parametrize("name,T,n,k,std,step,rounds", SIGN_CASES)
def test_route_sign_parity(name, T, n, k, std, step, rounds):
    announce(f"sign {name} T={T} n={n} k={k} step={step} rounds={rounds}")
    s = scores(T, n, std)
    ref = qb.sign_update(s, k, step, rounds)
    got = gpu_sign(s, k, step, rounds)
    assert (got["idx"] == ref["idx"]).all()
    assert (got["loads"] == ref["loads"]).all()
    assert (got["bias"] == ref["bias"]).all()
    assert tuple(int(v) for v in got["info"]) == tuple(ref["info"])
    assert np.allclose(got["w"], ref["w"], rtol=(k + 1) * 2.0 ** -24, atol=0)


def test_route_sign_two_experts_closed_form():
    # n = 2, k = 1, one token preferring expert 1 by D grid units: balance
    # after ceil(D / 2g) updates (the oracle's pin), here on the GPU
    s = np.array([[0.25, 0.25 + 3 * 2.0 ** -6]], np.float32)
    D = int(qb.to_fixed(s)[0, 1] - qb.to_fixed(s)[0, 0])
    g = 1 << 30
    got = gpu_sign(s, 1, g * 2.0 ** -40, 10000)
    assert int(got["info"][0]) == -(-D // (2 * g)) and int(got["info"][1]) == 0
    assert got["idx"][0, 0] == 0
