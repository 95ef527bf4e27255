"""Quantile Balancing (QB) routing -- oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain NumPy, integer
arithmetic for every routing decision, float64 for the mixture weights.

What the pages fix
------------------
* Routing: sigmoid scores on the full-width token; a per-expert bias
  (``e_score_correction_bias``) is added to the scores to pick the top-k
  experts; the mixture weights are the *raw* scores of the chosen experts,
  renormalised; the bias influences selection only
  ([K3-structure-5] Q&A "Stable LatentMoE 中，路由是如何工作的？";
  [K3-LatentMoE] Quantile Balancing paragraph).
* QB: a per-expert bias gives every expert exactly its target load, taken
  from the (1 - k/n) quantile of the expert's *margin* minus a common offset,
  with no step size ([K3-structure-5] Q&A "Quantile Balancing 是如何实现负载均衡的？").
* QB comes from the balanced-assignment problem and is coordinate descent
  on its dual that jumps to the exact coordinate minimiser, where
  DeepSeek-V3's fixed-step sign update is SignSGD on the same dual
  ([K3-structure-5] 延伸解读 "Quantile Balancing与DeepSeek-V3路由的异同").

Readings taken where the pages are open
--------------------------------------------------------------------
1. Exact arithmetic.  Scores are fp32; ``sfx = rint(s * 2^40)`` is exact for
   s >= 2^-17.  A bias is an int64 on the same 2^-40 grid.  The comparison
   key of (token t, expert e) is ``((sfx + bfx_e + 2^51) << 10) | (1023 - e)``:
   integer order is "higher biased score first, then lower expert index", so
   the k chosen experts of a token are always well defined.
2. Targets.  ``C_e = floor(T*k/n) + [e < (T*k mod n)]`` (the pages assume
   T*k/n is an integer; lower expert indices take the ceiling otherwise).
3. Margin.  For token t and expert e, the margin is e's unbiased key minus
   the k-th largest key among the *other* experts of t; t picks e at bias b
   exactly when ``margin + 1024*b > 0``.  Taking b as minus the midpoint of
   the C_e-th and (C_e+1)-th largest margins gives expert e exactly C_e
   tokens with the other biases held fixed: the exact coordinate minimiser
   of the dual, i.e. "minus the (1-C_e/T) quantile of the margin".
4. Schedule.  Coordinate rounds update every unbalanced expert at once from
   the same state (the lazy rule: balanced experts do not move).  Measured on
   the workloads here, coordinate steps alone (in parallel *or* one expert at
   a time) stall with a handful of experts off by one: the dual is piecewise
   linear and coordinate descent jams on it.  The rounds therefore stop once
   the count of unbalanced experts has not reached a new minimum for
   ``stall_rounds`` rounds, and exact balance is completed by shortest
   augmenting paths on the same dual (:func:`sap_step`): a move of several
   biases at once that transfers one unit of load from an overloaded to an
   underloaded expert through a chain of token swaps.  Any bias that
   balances every expert yields the *same* selection (see
   :func:`assignment_objective`), so the completion step changes no routing
   result, only how it is reached.
   The returned bias does depend on the schedule, which is fixed by these
   parameters: every unbalanced expert updated in each round from the same
   start-of-round biases; stall window ``stall_rounds = 3`` (a round that
   does not bring the unbalanced count below its best so far adds one; the
   third in a row ends the rounds); at most ``max_rounds = 64`` rounds and
   ``max_sap = 4096`` moves; each move takes the nearest underloaded expert
   (ties: lowest index) and its path of lowest predecessors.  The edge-cost
   bound of the sparse relaxation (start 2^30, x16 per retry, full
   relaxation past 2^44) changes no result.
5. Common offset.  After balancing, ``floor(sum(bfx)/n)`` is subtracted from
   every bias; selection is unchanged (every key of a token moves together).
6. Output order.  ``idx[t]`` lists the chosen experts by descending raw score,
   ties to the lower index; ``w[t, j] = s[t, idx_j] / sum_j s[t, idx_j]``.
"""
from __future__ import annotations

import numpy as np

FRAC_BITS = 40
IDX_BITS = 10
MAX_EXPERTS = 1 << IDX_BITS
KEY_OFFSET = 1 << 51
BIAS_LIMIT = 1 << 50          # |bias| < 1024 in score units
DIST_INF = 1 << 52            # path lengths at or above this are "unreachable"
PACKED_INF = DIST_INF << IDX_BITS

STATUS_OK = 0
STATUS_NOT_BALANCED = 1
STATUS_BIAS_RANGE = 2

MODE_FROZEN = 0
MODE_BATCH = 1


def targets(T: int, n: int, k: int) -> np.ndarray:
    """Per-expert target loads C_e (reading 2); they sum to T*k."""
    C = np.full(n, (T * k) // n, dtype=np.int64)
    C[: (T * k) % n] += 1
    return C


def to_fixed(scores: np.ndarray) -> np.ndarray:
    """fp32 scores -> int64 on the 2^-40 grid, round half to even (reading 1)."""
    s = np.asarray(scores, dtype=np.float32).astype(np.float64)
    return np.rint(s * 2.0 ** FRAC_BITS).astype(np.int64)


def bias_to_fixed(bias) -> np.ndarray:
    return np.rint(np.asarray(bias, dtype=np.float64) * 2.0 ** FRAC_BITS).astype(np.int64)


def fixed_to_bias(bfx: np.ndarray) -> np.ndarray:
    return np.asarray(bfx, dtype=np.int64).astype(np.float64) * 2.0 ** -FRAC_BITS


def packed_keys(sfx: np.ndarray, bfx: np.ndarray) -> np.ndarray:
    n = sfx.shape[1]
    e = np.arange(n, dtype=np.int64)
    return ((sfx + bfx[None, :] + KEY_OFFSET) << IDX_BITS) | (MAX_EXPERTS - 1 - e)


def select(sfx: np.ndarray, bfx: np.ndarray, k: int):
    """Top-k of the biased keys of every token.

    Returns (th_k, th_k1, S): the k-th and (k+1)-th largest key per token and
    the boolean selection matrix.  With k == n the (k+1)-th key is a sentinel
    below every key.
    """
    T, n = sfx.shape
    K = packed_keys(sfx, bfx)
    if T == 0:
        z = np.zeros(0, dtype=np.int64)
        return z, z, np.zeros((0, n), dtype=bool)
    if k < n:
        part = np.partition(K, (n - k - 1, n - k), axis=1)
        th_k, th_k1 = part[:, n - k].copy(), part[:, n - k - 1].copy()
    else:
        th_k, th_k1 = K.min(axis=1), np.zeros(T, dtype=np.int64)
    return th_k, th_k1, K >= th_k[:, None]


def margins(sfx_col: np.ndarray, e: int, S_col: np.ndarray, th_k, th_k1) -> np.ndarray:
    """Margin of expert e on every token (reading 3), in key units."""
    base = ((sfx_col + KEY_OFFSET) << IDX_BITS) | (MAX_EXPERTS - 1 - e)
    return base - np.where(S_col, th_k1, th_k)


def coordinate_bias(M: np.ndarray, C: int) -> int:
    """Exact coordinate minimiser for one expert: minus the midpoint between
    the C-th and (C+1)-th largest margins (floor division, exact integers)."""
    T = M.shape[0]
    Ms = np.sort(M)[::-1]
    if C == 0:
        return -(int(Ms[0]) >> IDX_BITS) - 1
    if C == T:
        return -(int(Ms[T - 1]) >> IDX_BITS) + 1
    return -((int(Ms[C - 1]) + int(Ms[C])) >> (IDX_BITS + 1))


def coordinate_round(sfx, bfx, k, C, state=None):
    """One QB round: every unbalanced expert jumps to its exact coordinate
    minimiser, all computed from the same (start-of-round) biases."""
    th_k, th_k1, S = state if state is not None else select(sfx, bfx, k)
    L = S.sum(axis=0)
    new = bfx.copy()
    for e in np.nonzero(L != C)[0]:
        M = margins(sfx[:, e], int(e), S[:, e], th_k, th_k1)
        new[e] = coordinate_bias(M, int(C[e]))
    return new


def _relax_rows(d, Kp_rows, S_rows):
    """Best packed candidate (distance << 10 | predecessor) for every (row, B)
    with B not chosen by the row's token, from the current distances d.

    Candidate for B through token t: min over chosen A of d_A + rho_t(A, B),
    predecessor = the lowest A attaining it.  rho_t(A, B) = (sfx_tA + b_A) -
    (sfx_tB + b_B) - [A > B].
    """
    R, n = Kp_rows.shape
    reach = d < DIST_INF
    BIG = np.int64(1 << 62)
    V = np.where(S_rows & reach[None, :], d[None, :] + Kp_rows, BIG)
    v1 = V.min(axis=1)
    a1 = np.argmin(V, axis=1).astype(np.int64)
    ok = v1 < BIG
    B = np.arange(n, dtype=np.int64)[None, :]
    val = v1[:, None] - (a1[:, None] > B)
    pred = np.broadcast_to(a1[:, None], (R, n)).copy()
    # Rows where two chosen experts share the minimum: apply the general rule
    # (value v1 - 1 with the lowest tied A above B, else v1 with the lowest A
    # reaching v1 from either tie class).
    ties = np.nonzero(ok & ((V == v1[:, None]).sum(axis=1) > 1))[0]
    for r in ties:
        E1 = np.nonzero(V[r] == v1[r])[0]
        E2 = np.nonzero(V[r] == v1[r] + 1)[0]
        for b in range(n):
            above = E1[E1 > b]
            if above.size:
                val[r, b], pred[r, b] = v1[r] - 1, above.min()
            else:
                cands = np.concatenate([E1, E2[E2 > b]])
                val[r, b], pred[r, b] = v1[r], cands.min()
    cand = val - Kp_rows
    valid = ok[:, None] & ~S_rows & (cand < DIST_INF)
    return np.where(valid, (cand << IDX_BITS) | pred, PACKED_INF)


def shortest_paths(sfx, bfx, S, over, under):
    """Bellman-Ford over experts from every overloaded expert.

    Edge A -> B exists through token t when t currently picks A and not B;
    its length is the reduced cost rho_t(A, B) >= 0, the relative bias change
    (grid units) that moves t from A to B.  Returns packed
    (distance << 10 | predecessor) per expert, ties to the lowest
    predecessor.  Each pass relaxes the tokens that choose an expert whose
    distance changed in the previous pass; the passes stop once no expert at
    or below D* (the distance of the nearest underloaded expert) changed, at
    which point every distance <= D* and its predecessor are final.
    """
    T, n = sfx.shape
    ar = np.arange(n, dtype=np.int64)
    packed = np.where(over, ar, PACKED_INF).astype(np.int64)
    changed = over.copy()
    while True:
        rows = np.nonzero(S[:, changed].any(axis=1))[0]
        new = packed
        if rows.size:
            Kp = sfx[rows] + bfx[None, :]
            cp = _relax_rows(packed >> IDX_BITS, Kp, S[rows])
            new = np.minimum(packed, cp.min(axis=0))
        D = np.where(under, new >> IDX_BITS, DIST_INF).min(initial=DIST_INF)
        changed = new != packed
        packed = new
        if not (changed & ((packed >> IDX_BITS) <= D)).any():
            return packed


def sparse_edges(sfx, bfx, S, th_k, th_k1, delta):
    """Every (token t, chosen A, unchosen B) with rho_t(A, B) <= delta, as
    arrays (A, B, rho).  A path no longer than delta uses only such edges, so
    distances up to delta computed on this list are exact."""
    T, n = sfx.shape
    Kp = sfx + bfx[None, :]
    kpk = (th_k >> IDX_BITS) - KEY_OFFSET
    kpk1 = (th_k1 >> IDX_BITS) - KEY_OFFSET
    rows = np.nonzero(kpk - kpk1 <= delta + 1)[0]
    As, Bs, Rs = [], [], []
    for t in rows:
        low = np.nonzero(S[t] & (Kp[t] - kpk[t] <= delta + 1))[0]
        high = np.nonzero(~S[t] & (kpk1[t] - Kp[t] <= delta + 1))[0]
        if low.size == 0 or high.size == 0:
            continue
        A = np.repeat(low, high.size)
        B = np.tile(high, low.size)
        rho = Kp[t, A] - Kp[t, B] - (A > B)
        keep = rho <= delta
        As.append(A[keep]); Bs.append(B[keep]); Rs.append(rho[keep])
    if not As:
        z = np.zeros(0, np.int64)
        return z, z, z
    return (np.concatenate(As).astype(np.int64), np.concatenate(Bs).astype(np.int64),
            np.concatenate(Rs).astype(np.int64))


def shortest_paths_edges(A, B, rho, over, under):
    """Bellman-Ford on an explicit edge list with the same packing, tie rule
    and stopping rule as :func:`shortest_paths`."""
    n = over.shape[0]
    packed = np.where(over, np.arange(n, dtype=np.int64), PACKED_INF).astype(np.int64)
    while True:
        d = packed >> IDX_BITS
        dA = d[A]
        ok = dA < DIST_INF
        cand = dA + rho
        ok &= cand < DIST_INF
        new = packed.copy()
        np.minimum.at(new, B[ok], (cand[ok] << IDX_BITS) | A[ok])
        D = np.where(under, new >> IDX_BITS, DIST_INF).min(initial=DIST_INF)
        changed = new != packed
        packed = new
        if not (changed & ((packed >> IDX_BITS) <= D)).any():
            return packed


SPARSE_DELTA = 1 << 30        # first edge-cost bound of the sparse relaxation
SPARSE_DELTA_MAX = 1 << 44    # beyond it the full relaxation is used


def sap_step(sfx, bfx, k, C, state=None, sparse=True):
    """One shortest-augmenting-path move on the dual (reading 4).

    Lowers every expert's bias by (D* - min(d, D*)), which keeps every token's
    selection valid and makes the shortest path from an overloaded expert to
    the nearest underloaded expert u* tight, then raises the i-th expert on
    that path by i grid units so that each path token moves one step along
    it.  Returns the new biases, or None when no underloaded expert is
    reachable.  With ``sparse`` the distances come from the edges of reduced
    cost <= delta (delta grows 16x until D* <= delta), which gives the same
    distances and predecessors up to D* as the full relaxation; once delta
    has passed SPARSE_DELTA_MAX without reaching D*, the full relaxation
    decides.  The result therefore never depends on delta.
    """
    th_k, th_k1, S = state if state is not None else select(sfx, bfx, k)
    L = S.sum(axis=0)
    over, under = L > C, L < C
    packed = None
    if sparse:
        delta = SPARSE_DELTA
        while delta <= SPARSE_DELTA_MAX:
            A, B, rho = sparse_edges(sfx, bfx, S, th_k, th_k1, delta)
            cand = shortest_paths_edges(A, B, rho, over, under)
            D = int(np.where(under, cand >> IDX_BITS, DIST_INF).min())
            if D <= delta:
                packed = cand
                break
            delta *= 16
    if packed is None:
        packed = shortest_paths(sfx, bfx, S, over, under)
    d = packed >> IDX_BITS
    pred = packed & (MAX_EXPERTS - 1)
    d_under = np.where(under, d, DIST_INF)
    D = int(d_under.min())
    if D >= DIST_INF:
        return None
    u = int(np.argmin(d_under))
    path = [u]
    while not over[path[-1]]:
        path.append(int(pred[path[-1]]))
        if len(path) > len(C) + 1:
            return None
    path.reverse()
    new = bfx + (np.minimum(d, D) - D)
    for i, v in enumerate(path):
        new[v] += i
    return new


def route_qb(scores, k, bias=None, mode=MODE_BATCH, max_rounds=64, stall_rounds=3,
             max_sap=4096):
    """Route a batch of fp32 scores [T, n] to k experts per token.

    Returns a dict with ``idx`` [T,k] int32, ``w`` [T,k] float64, ``loads``
    [n] int64, ``bias`` [n] float64 (exact on the 2^-40 grid), ``bfx`` [n]
    int64 and ``info`` = (coordinate rounds, status, max |L - C|,
    augmenting-path moves).
    """
    s = np.asarray(scores, dtype=np.float32)
    T, n = s.shape
    if not (1 <= k <= n <= MAX_EXPERTS):
        raise ValueError("need 1 <= k <= n <= 1024")
    if T and not (np.isfinite(s).all() and (s >= 0).all() and (s <= 1).all()):
        raise ValueError("scores must lie in [0, 1]")
    sfx = to_fixed(s)
    bfx = np.zeros(n, np.int64) if bias is None else bias_to_fixed(bias)
    if np.abs(bfx).max(initial=0) >= BIAS_LIMIT:
        raise ValueError("bias out of range")
    C = targets(T, n, k)
    rounds = sap_moves = 0
    status = STATUS_OK

    def in_range(b):
        return np.abs(b).max(initial=0) < BIAS_LIMIT

    state = select(sfx, bfx, k)
    if mode == MODE_BATCH:
        best, since_best = None, 0
        while True:
            L = state[2].sum(axis=0)
            imb = int((L != C).sum())
            if imb == 0 or rounds >= max_rounds:
                break
            if best is None or imb < best:
                best, since_best = imb, 0
            else:
                since_best += 1
                if since_best >= stall_rounds:
                    break
            bfx = coordinate_round(sfx, bfx, k, C, state)
            rounds += 1
            if not in_range(bfx):
                status = STATUS_BIAS_RANGE
                break
            state = select(sfx, bfx, k)
        while status == STATUS_OK:
            L = state[2].sum(axis=0)
            if (L == C).all():
                break
            if sap_moves >= max_sap:
                status = STATUS_NOT_BALANCED
                break
            nb = sap_step(sfx, bfx, k, C, state)
            if nb is None:
                status = STATUS_NOT_BALANCED
                break
            bfx = nb
            sap_moves += 1
            if not in_range(bfx):
                status = STATUS_BIAS_RANGE
                break
            state = select(sfx, bfx, k)
        if status == STATUS_OK:
            bfx = bfx - (int(bfx.sum()) // n)
            state = select(sfx, bfx, k)
    S = state[2]
    L = S.sum(axis=0).astype(np.int64)
    residual = int(np.abs(L - C).max(initial=0))
    idx, w = ordered_outputs(s, sfx, S, k)
    return dict(idx=idx, w=w, loads=L, bias=fixed_to_bias(bfx), bfx=bfx,
                info=(rounds, status, residual, sap_moves))


def step_to_fixed(step) -> int:
    """A bias step in score units on the 2^-40 grid (round half to even)."""
    v = int(np.rint(np.float64(step) * (1 << FRAC_BITS)))
    if v <= 0 or v >= BIAS_LIMIT:
        raise ValueError("step must be positive and below the bias range")
    return v


def sign_update(scores, k, step, max_rounds, bias=None):
    """DeepSeek-V3's bias rule run on one batch, as the baseline QB is
    compared with: each round takes the top-k under the current bias and
    moves every expert's bias by a fixed step towards its target load,
    b_e += step * sign(C_e - L_e), until every load equals its target or
    ``max_rounds`` updates were made.  The pages describe it as sign descent
    (SignSGD) on the same dual objective whose exact coordinate minimiser QB
    takes, with a step that has to be tuned by hand ([K3-structure-5]
    延伸解读 "Quantile Balancing与DeepSeek-V3路由的异同").  The same exact keys and
    targets as :func:`route_qb`; no common offset is removed.

    Returns the dict of :func:`route_qb` with ``info`` = (updates, status,
    max |L - C|, 0): status 0 balanced, 1 not balanced after ``max_rounds``,
    2 bias out of range.
    """
    s = np.asarray(scores, dtype=np.float32)
    T, n = s.shape
    if not (1 <= k <= n <= MAX_EXPERTS):
        raise ValueError("need 1 <= k <= n <= 1024")
    if max_rounds < 0:
        raise ValueError("max_rounds must be >= 0")
    sfx = to_fixed(s)
    bfx = np.zeros(n, np.int64) if bias is None else bias_to_fixed(bias)
    if np.abs(bfx).max(initial=0) >= BIAS_LIMIT:
        raise ValueError("bias out of range")
    g = step_to_fixed(step)
    C = targets(T, n, k)
    rounds, status = 0, STATUS_OK
    state = select(sfx, bfx, k)
    while True:
        L = state[2].sum(axis=0)
        if (L == C).all():
            break
        if rounds >= max_rounds:
            status = STATUS_NOT_BALANCED
            break
        bfx = bfx + g * np.sign(C - L).astype(np.int64)
        rounds += 1
        if np.abs(bfx).max(initial=0) >= BIAS_LIMIT:
            status = STATUS_BIAS_RANGE
            break
        state = select(sfx, bfx, k)
    S = state[2]
    L = S.sum(axis=0).astype(np.int64)
    idx, w = ordered_outputs(s, sfx, S, k)
    return dict(idx=idx, w=w, loads=L, bias=fixed_to_bias(bfx), bfx=bfx,
                info=(rounds, status, int(np.abs(L - C).max(initial=0)), 0))


def ordered_outputs(s, sfx, S, k):
    """Chosen experts per token by descending raw score (ties: lower index),
    and the raw scores renormalised over the chosen k (reading 6)."""
    T, n = s.shape
    e = np.arange(n, dtype=np.int64)
    order_key = np.where(S, (((1 << FRAC_BITS) - sfx) << IDX_BITS) | e, np.int64(1 << 62))
    idx = np.argsort(order_key, axis=1, kind="stable")[:, :k].astype(np.int32)
    raw = np.take_along_axis(s.astype(np.float64), idx.astype(np.int64), axis=1)
    w = raw / raw.sum(axis=1, keepdims=True) if T else raw
    return idx, w


def plain_topk(scores, k):
    """Top-k of the raw scores with the same tie rule, no bias."""
    s = np.asarray(scores, dtype=np.float32)
    sfx = to_fixed(s)
    _, _, S = select(sfx, np.zeros(s.shape[1], np.int64), k)
    return S


def assignment_objective(scores, S) -> int:
    """The quantity a balanced bias-based selection maximises, exactly.

    For any bias b with loads equal to C, summing the per-token top-k
    inequalities of the keys and cancelling sum_e b_e*C_e (the same for every
    balanced selection) shows that the selection maximises
    F(S) = sum over chosen (t, e) of (1024*sfx[t,e] - e), strictly.  So the
    balanced selection is the unique maximiser of F over all selections with
    k experts per token and load C_e per expert.
    """
    sfx = to_fixed(scores)
    t, e = np.nonzero(S)
    return int(sum(1024 * int(v) for v in sfx[t, e])) - int(e.sum())
