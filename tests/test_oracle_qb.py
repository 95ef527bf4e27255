"""Pins of the QB routing oracle against what the pages and mathematics fix.

Each pin is chosen so that a plausible mistake in ``oracle.qb`` (a wrong sign,
an off-by-one order statistic, a dropped tie rule, a transposed index) fails:

* brute force over every balanced assignment on tiny inputs,
* the LP optimum of the balanced-assignment problem (totally unimodular, so
  the LP optimum is the integral optimum) -- the problem QB starts from,
* k = 1 against the textbook Hungarian algorithm with expert slots replicated,
* dual optimality, the fixed-point (idempotence) property, the coordinate
  step, the DeepSeek-V3 sign-update relation, the weights' definition and
  the degenerate cases.
"""
import itertools

import numpy as np
import pytest
from scipy.optimize import linear_sum_assignment, linprog

from oracle import qb


def rand_scores(T, n, seed, skew=0.5):
    rng = np.random.default_rng(seed)
    logits = rng.standard_normal((T, n)) + skew * rng.standard_normal(n)[None, :]
    return (1 / (1 + np.exp(-logits))).astype(np.float32)


def sel_matrix(idx, n):
    S = np.zeros((idx.shape[0], n), bool)
    np.put_along_axis(S, idx.astype(np.int64), True, axis=1)
    return S


def test_targets_sum_and_spread():
    for T, n, k in [(64, 32, 4), (4096, 896, 16), (64, 896, 16), (5, 3, 2), (0, 7, 3)]:
        C = qb.targets(T, n, k)
        assert C.sum() == T * k
        assert set(np.unique(C)) <= {T * k // n, -(-T * k // n)}
        assert (np.diff(C) <= 0).all()       # ceilings go to the lowest indices


def test_fixed_point_exact_for_normal_scores():
    s = np.array([0.5, 0.75, 2.0 ** -17, 1.0, 0.0, 0.1], np.float32)
    sfx = qb.to_fixed(s[None, :])[0]
    assert list(sfx[:5]) == [2 ** 39, 3 * 2 ** 38, 2 ** 23, 2 ** 40, 0]
    assert sfx[5] == round(float(np.float32(0.1)) * 2 ** 40)


@pytest.mark.parametrize("T,n,k,seed", [(6, 4, 2, s) for s in range(4)] +
                         [(5, 3, 2, s) for s in range(3)] + [(5, 5, 2, 7)])
def test_brute_force(T, n, k, seed):
    s = rand_scores(T, n, seed, skew=1.0)
    r = qb.route_qb(s, k)
    assert r["info"][1] == qb.STATUS_OK
    C = qb.targets(T, n, k)
    best, best_S = None, None
    choices = list(itertools.combinations(range(n), k))
    for combo in itertools.product(choices, repeat=T):
        S = np.zeros((T, n), bool)
        for t, c in enumerate(combo):
            S[t, list(c)] = True
        if not (S.sum(0) == C).all():
            continue
        F = qb.assignment_objective(s, S)
        if best is None or F > best:
            best, best_S = F, S
    got = sel_matrix(r["idx"], n)
    assert (got == best_S).all()
    assert (r["loads"] == C).all()


@pytest.mark.parametrize("T,n,k,seed", [(256, 16, 4, 0), (300, 24, 5, 1)])
def test_lp_optimum(T, n, k, seed):
    s = rand_scores(T, n, seed)
    r = qb.route_qb(s, k)
    assert r["info"][1] == qb.STATUS_OK
    C = qb.targets(T, n, k)
    # maximise sum x*s s.t. row sums k, column sums C, 0 <= x <= 1
    A_eq = np.zeros((T + n, T * n))
    for t in range(T):
        A_eq[t, t * n:(t + 1) * n] = 1
    for e in range(n):
        A_eq[T + e, e::n] = 1
    b_eq = np.concatenate([np.full(T, k), C])
    res = linprog(-s.astype(np.float64).ravel(), A_eq=A_eq, b_eq=b_eq, bounds=(0, 1),
                  method="highs")
    assert res.status == 0
    x = res.x.reshape(T, n)
    assert np.abs(x - np.round(x)).max() < 1e-6
    got = sel_matrix(r["idx"], n)
    assert (got == (x > 0.5)).all()


def lp_selection(s, k):
    """The balanced-assignment LP (sparse constraints): row sums k, column
    sums C, 0 <= x <= 1, maximise sum x*s.  Totally unimodular, so the HiGHS
    vertex is integral; returns the boolean selection."""
    from scipy.sparse import coo_matrix
    T, n = s.shape
    C = qb.targets(T, n, k)
    t_idx = np.repeat(np.arange(T), n)
    e_idx = np.tile(np.arange(n), T)
    cols = np.arange(T * n)
    A_eq = coo_matrix((np.ones(2 * T * n), (np.concatenate([t_idx, T + e_idx]),
                                             np.concatenate([cols, cols]))),
                      shape=(T + n, T * n)).tocsr()
    b_eq = np.concatenate([np.full(T, k), C])
    res = linprog(-s.astype(np.float64).ravel(), A_eq=A_eq, b_eq=b_eq, bounds=(0, 1),
                  method="highs")
    assert res.status == 0
    x = res.x.reshape(T, n)
    assert np.abs(x - np.round(x)).max() < 1e-6
    return x > 0.5


@pytest.mark.parametrize("max_rounds", [64, 1, 0])
def test_lp_optimum_independent_of_schedule(max_rounds):
    """The LP solved from scratch at T=600, n=32, k=4: the selection must be
    its optimum whether balance comes mostly from quantile rounds or mostly
    (max_rounds 1, 0) from augmenting paths."""
    T, n, k = 600, 32, 4
    s = rand_scores(T, n, 41, skew=0.7)
    r = qb.route_qb(s, k, max_rounds=max_rounds)
    assert r["info"][1] == qb.STATUS_OK
    if max_rounds < 64:
        assert r["info"][3] > 20          # many moves: the schedule differs
    assert (sel_matrix(r["idx"], n) == lp_selection(s, k)).all()


@pytest.mark.parametrize("max_rounds", [64, 0])
def test_k1_hungarian_large(max_rounds):
    """k = 1 at T=2000, n=64 against the textbook assignment solver with
    expert slots replicated (no token can take two slots of one expert when
    k = 1, so the assignment problem is exactly the balanced routing)."""
    T, n = 2000, 64
    s = rand_scores(T, n, 43, skew=0.7)
    r = qb.route_qb(s, 1, max_rounds=max_rounds)
    assert r["info"][1] == qb.STATUS_OK
    C = qb.targets(T, n, 1)
    slots = np.repeat(np.arange(n), C)
    rows, cols = linear_sum_assignment(-s.astype(np.float64)[:, slots])
    assert (r["idx"][:, 0] == slots[cols[np.argsort(rows)]]).all()


def test_selection_same_across_schedules_k3_like():
    """T=2000, n=64, k=4: quantile rounds, a round cap of 2 and pure
    augmenting paths reach different biases but the same selection, and
    each bias certifies it (the selection is the top-k under it and every
    load equals its target)."""
    T, n, k = 2000, 64, 4
    s = rand_scores(T, n, 41, skew=0.7)
    sfx = qb.to_fixed(s)
    C = qb.targets(T, n, k)
    runs = [qb.route_qb(s, k, max_rounds=m) for m in (64, 2, 0)]
    assert len({tuple(r["bfx"]) for r in runs}) > 1
    for r in runs:
        assert r["info"][1] == qb.STATUS_OK
        S = sel_matrix(r["idx"], n)
        assert (S == sel_matrix(runs[0]["idx"], n)).all()
        K = qb.packed_keys(sfx, r["bfx"])
        kth = -np.sort(-K, axis=1)[:, k - 1]
        assert (S == (K >= kth[:, None])).all() and (S.sum(0) == C).all()


def test_sap_sparse_falls_back_to_full_relaxation():
    """A start bias that makes the only augmenting path longer than the
    sparse bound (about 100 score units against 2^44 grid units = 16): the
    sparse step must hand over to the full relaxation and move exactly as it
    does."""
    T, n, k = 40, 3, 1
    s = rand_scores(T, n, 5, skew=0.2)
    sfx = qb.to_fixed(s)
    C = qb.targets(T, n, k)
    b = np.array([0, -100 << 40, -100 << 40], np.int64)   # expert 0 takes every token
    st = qb.select(sfx, b, k)
    assert st[2][:, 0].all()
    full = qb.sap_step(sfx, b, k, C, st, sparse=False)
    fast = qb.sap_step(sfx, b, k, C, st, sparse=True)
    assert full is not None and (fast == full).all()
    # the move is a real one: expert 0 drops one token, one underloaded expert gains it
    L = qb.select(sfx, full, k)[2].sum(0)
    assert L[0] == T - 1 and sorted(L[1:]) == [0, 1]
    # and the whole loop, from that start, still reaches the LP optimum
    r = qb.route_qb(s, k, bias=qb.fixed_to_bias(b), max_rounds=0)
    assert r["info"][1] == qb.STATUS_OK
    assert (sel_matrix(r["idx"], n) == lp_selection(s, k)).all()


def test_k1_hungarian():
    T, n = 60, 12
    s = rand_scores(T, n, 3, skew=1.0)
    r = qb.route_qb(s, 1)
    C = qb.targets(T, n, 1)
    slots = np.repeat(np.arange(n), C)
    rows, cols = linear_sum_assignment(-s.astype(np.float64)[:, slots])
    ref = slots[cols[np.argsort(rows)]]
    assert (r["idx"][:, 0] == ref).all()


def dual_value(sfx, bfx, C, k):
    """D(b) = sum_t (sum of the k largest s+b of token t) - sum_e C_e b_e,
    exact integers on the 2^-40 grid."""
    v = sfx + bfx[None, :]
    top = -np.sort(-v, axis=1)[:, :k]
    return int(sum(int(x) for x in top.sum(axis=1))) - int(sum(int(c) * int(b) for c, b in zip(C, bfx)))


def test_dual_optimality_and_sign_update():
    T, n, k = 200, 16, 3
    s = rand_scores(T, n, 11, skew=1.0)
    r = qb.route_qb(s, k)
    sfx = qb.to_fixed(s)
    C = qb.targets(T, n, k)
    b = r["bfx"]
    D0 = dual_value(sfx, b, C, k)
    rng = np.random.default_rng(0)
    for _ in range(50):
        delta = rng.integers(-2 ** 30, 2 ** 30, size=n)
        assert dual_value(sfx, b + delta, C, k) >= D0
    # DeepSeek-V3's sign rule is SignSGD on the same dual: from an unbalanced
    # bias, the slope of D along e_e is L_e - C_e, and b + g*sign(C - L)
    # with a small step g lowers D by g * sum |L - C|.
    b0 = np.zeros(n, np.int64)
    _, _, S0 = qb.select(sfx, b0, k)
    L0 = S0.sum(0)
    assert (L0 != C).any()
    g = 1
    step = np.sign(C - L0)
    _, _, S1 = qb.select(sfx, b0 + g * step, k)
    assert (S1 == S0).all()                  # no key crossed for so small a step
    assert dual_value(sfx, b0 + g * step, C, k) - dual_value(sfx, b0, C, k) == -g * int(np.abs(L0 - C).sum())
    for e in range(n):
        one = np.zeros(n, np.int64)
        one[e] = 1
        assert dual_value(sfx, b0 + one, C, k) - dual_value(sfx, b0, C, k) == L0[e] - C[e]


def test_idempotent_fixed_point():
    s = rand_scores(512, 32, 5)
    r1 = qb.route_qb(s, 4)
    r2 = qb.route_qb(s, 4, bias=r1["bias"])
    assert r2["info"][0] == 0 and r2["info"][3] == 0
    assert (r2["bfx"] == r1["bfx"]).all()
    assert (r2["idx"] == r1["idx"]).all()
    assert 0 <= int(r1["bfx"].sum()) < 32        # common offset removed


def test_coordinate_step_is_exact():
    T, n, k = 500, 20, 3
    s = rand_scores(T, n, 8, skew=1.0)
    sfx = qb.to_fixed(s)
    C = qb.targets(T, n, k)
    rng = np.random.default_rng(1)
    b = rng.integers(-2 ** 36, 2 ** 36, size=n)
    th_k, th_k1, S = qb.select(sfx, b, k)
    for e in range(n):
        M = qb.margins(sfx[:, e], e, S[:, e], th_k, th_k1)
        b2 = b.copy()
        b2[e] = qb.coordinate_bias(M, int(C[e]))
        _, _, S2 = qb.select(sfx, b2, k)
        assert S2[:, e].sum() == C[e]


def test_zero_bias_is_plain_topk_and_weights():
    T, n, k = 100, 24, 5
    s = rand_scores(T, n, 2)
    r = qb.route_qb(s, k, mode=qb.MODE_FROZEN)
    # plain top-k by raw score, ties to the lower index, written independently
    order = np.lexsort((np.broadcast_to(np.arange(n), (T, n)), -s.astype(np.float64)), axis=1)
    assert (r["idx"] == order[:, :k]).all()
    raw = np.take_along_axis(s.astype(np.float64), r["idx"].astype(np.int64), 1)
    assert np.allclose(r["w"].sum(1), 1.0, atol=1e-15)
    assert np.allclose(r["w"], raw / raw.sum(1, keepdims=True), rtol=1e-15)
    # a constant bias changes nothing
    r2 = qb.route_qb(s, k, bias=np.full(n, 0.125), mode=qb.MODE_FROZEN)
    assert (r2["idx"] == r["idx"]).all()


def test_weights_do_not_depend_on_bias():
    T, n, k = 300, 16, 4
    s = rand_scores(T, n, 4, skew=1.5)
    r = qb.route_qb(s, k)
    plain = qb.route_qb(s, k, mode=qb.MODE_FROZEN)
    assert not (r["idx"] == plain["idx"]).all()                 # skew: bias moved selection
    assert np.ptp(r["bias"]) > 0
    raw = np.take_along_axis(s.astype(np.float64), r["idx"].astype(np.int64), 1)
    assert np.allclose(r["w"], raw / raw.sum(1, keepdims=True), rtol=1e-15)
    # idx order: descending raw score
    assert (np.diff(raw, axis=1) <= 0).all()


def test_balanced_input_keeps_zero_bias():
    n = 16
    T = 4 * n
    rng = np.random.default_rng(0)
    s = (0.1 * rng.random((T, n))).astype(np.float32)
    for t in range(T):
        s[t, t % n] = 0.9
    r = qb.route_qb(s, 1)
    assert r["info"][0] == 0 and r["info"][3] == 0
    assert (r["bfx"] == 0).all()
    assert (r["idx"][:, 0] == np.arange(T) % n).all()


def test_degenerate_duplicate_tokens_report_not_balanced():
    s = np.tile(np.array([[0.7, 0.3]], np.float32), (4, 1))   # 4 identical tokens, C = (2, 2)
    r = qb.route_qb(s, 1, max_rounds=8, max_sap=8)
    assert r["info"][1] == qb.STATUS_NOT_BALANCED


def test_edge_cases():
    r = qb.route_qb(np.zeros((0, 8), np.float32), 2)
    assert r["idx"].shape == (0, 2) and (r["loads"] == 0).all() and r["info"][1] == 0
    s = rand_scores(10, 4, 0)
    r = qb.route_qb(s, 4)                 # k == n: everything chosen
    assert (r["loads"] == 10).all() and r["info"][1] == 0
    with pytest.raises(ValueError):
        qb.route_qb(s, 5)
    with pytest.raises(ValueError):
        qb.route_qb(np.full((2, 4), 1.5, np.float32), 1)


def test_qb_balances_skewed_batch():
    T, n, k = 1024, 64, 8
    s = rand_scores(T, n, 9, skew=1.0)
    r = qb.route_qb(s, k)
    assert r["info"][1] == qb.STATUS_OK
    assert (r["loads"] == qb.targets(T, n, k)).all()
    # the returned bias reproduces the selection in frozen mode
    f = qb.route_qb(s, k, bias=r["bias"], mode=qb.MODE_FROZEN)
    assert (f["idx"] == r["idx"]).all()


def test_sparse_paths_equal_full_relaxation():
    # the augmenting-path step on the edges of reduced cost <= delta must give
    # exactly the biases of the full Bellman-Ford relaxation
    for seed, (T, n, k) in enumerate([(400, 24, 3), (600, 40, 5), (300, 16, 2)]):
        s = rand_scores(T, n, 20 + seed, skew=1.0)
        sfx = qb.to_fixed(s)
        C = qb.targets(T, n, k)
        b = np.zeros(n, np.int64)
        for _ in range(3):
            b = qb.coordinate_round(sfx, b, k, C)
        moves = 0
        while moves < 6:
            st = qb.select(sfx, b, k)
            if (st[2].sum(0) == C).all():
                break
            full = qb.sap_step(sfx, b, k, C, st, sparse=False)
            fast = qb.sap_step(sfx, b, k, C, st, sparse=True)
            assert (full == fast).all()
            b = full
            moves += 1
        assert moves > 0


# --- the fixed-step sign update (DeepSeek-V3's bias rule) -----------------
# Pinned by closed forms: with n = 2, k = 1 and tokens that all prefer
# expert 1 by margins D_t (fixed-point units), the rule raises b_0 - b_1 by
# 2*g per round and token t switches once 2*g*r >= D_t (equal keys go to the
# lower index), so balance (C = (T/2, T/2)) comes after ceil(D_(T/2) / 2g)
# rounds, D_(T/2) the (T/2)-th smallest margin.

def _two_expert_scores(margins_fx):
    base = np.float32(0.25)
    s = np.empty((len(margins_fx), 2), np.float32)
    for t, m in enumerate(margins_fx):
        s[t, 0] = base
        s[t, 1] = np.float32(base + np.float64(m) * 2.0 ** -40)
    return s


def test_sign_update_two_experts_closed_form():
    for g_exp in (24, 30, 33):
        g = 1 << g_exp
        # one token: rounds = ceil(D / 2g)
        s = _two_expert_scores([3 * 2 ** 34])
        D = int(qb.to_fixed(s)[0, 1] - qb.to_fixed(s)[0, 0])
        r = qb.sign_update(s, 1, g * 2.0 ** -40, 10 ** 6)
        assert r["info"][:2] == (-(-D // (2 * g)), qb.STATUS_OK)
        assert r["bfx"][0] == -r["bfx"][1] == g * r["info"][0]
        assert r["idx"][0, 0] == 0 and r["loads"].tolist() == [1, 0]
    # four tokens, wide-apart margins: the second smallest decides
    s = _two_expert_scores([7 * 2 ** 36, 2 ** 33, 3 * 2 ** 35, 2 ** 38])
    sfx = qb.to_fixed(s)
    D = np.sort(sfx[:, 1] - sfx[:, 0])
    g = 1 << 31
    r = qb.sign_update(s, 1, g * 2.0 ** -40, 10 ** 6)
    assert r["info"][:3] == (-(-int(D[1]) // (2 * g)), qb.STATUS_OK, 0)
    assert r["loads"].tolist() == [2, 2]


def test_sign_update_exact_tie_goes_to_lower_index():
    g = 1 << 30
    s = _two_expert_scores([6 * g])  # D = 6g: keys equal after 3 rounds
    D = int(qb.to_fixed(s)[0, 1] - qb.to_fixed(s)[0, 0])
    assert D == 6 * g
    r = qb.sign_update(s, 1, g * 2.0 ** -40, 100)
    assert r["info"][0] == 3 and r["idx"][0, 0] == 0


def test_sign_update_balanced_input_and_round_cap():
    s = rand_scores(300, 16, 3)
    ref = qb.route_qb(s, 4)
    r = qb.sign_update(s, 4, 2.0 ** -10, 50, bias=ref["bias"])
    assert r["info"] == (0, qb.STATUS_OK, 0, 0)
    assert (r["bfx"] == ref["bfx"]).all() and (r["idx"] == ref["idx"]).all()
    # from zero: a capped run reports "not balanced" with its residual; the
    # balanced result, when reached, is the unique balanced selection
    r0 = qb.sign_update(s, 4, 2.0 ** -10, 0)
    assert r0["info"][0] == 0 and r0["info"][1] == qb.STATUS_NOT_BALANCED
    assert (r0["idx"] == qb.route_qb(s, 4, mode=qb.MODE_FROZEN)["idx"]).all()
    r5 = qb.sign_update(s, 4, 2.0 ** -10, 5)
    assert r5["info"][0] == 5 and r5["info"][1] == qb.STATUS_NOT_BALANCED
    assert r5["info"][2] == int(np.abs(r5["loads"] - qb.targets(300, 16, 4)).max())
