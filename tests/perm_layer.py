"""A layer whose weights are scaled permutation matrices, and its output
written out by hand.

With such weights every step of the Stable LatentMoE layer reduces to gathers
and scalar functions: z = x[sigma]; routed expert e: g = a_e z[pi_g,e],
u = b_e z[pi_u,e], y_e = c_e h[pi_d,e] with h = SiTU-GLU(g, u); the latent
sum over the chosen experts weighted by the renormalised raw scores;
RMSNorm with gain gamma; a scatter back to width d; plus the shared MLP on
the same pattern.  The router weights are zero, so every token's scores are
sigmoid(p) of the per-expert logit offsets, and top-2 picks experts 2 and 0.
Permutations (not identities) make a transposed operand visible; distinct
a, b, c per expert make a swapped gate/up, a wrong expert or a wrong weight
visible.
"""
import numpy as np

T, D, LAT, N, K, S = 5, 128, 64, 4, 2, 128
LOGIT_OFFSET = np.array([1.0, -0.5, 2.0, 0.3])
TOP = np.array([2, 0])
EPS = 1e-6


def _perm_matrix(rows, cols, src):
    """M[i, src[i]] = 1, so (M v)_i = v[src[i]]."""
    M = np.zeros((rows, cols))
    M[np.arange(rows), src] = 1.0
    return M


def build(seed=11, exact_mxfp4=False):
    """(inputs as float64 arrays keyed like the layer's weights, parameters)."""
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1.5, (T, D)).astype(np.float32).astype(np.float64)
    sigma = rng.permutation(D)[:LAT]
    if exact_mxfp4:   # {1, 1.5} x 2^j: exact in E2M1 x 2^E
        a, b, c = (np.array([1.5, 3.0, 0.75, 2.0]), np.array([3.0, 24.0, 12.0, 48.0]),
                   np.array([0.75, 1.5, 1.0, 2.0]))
    else:             # fp32-exact values
        a = rng.uniform(0.5, 3, N).astype(np.float32).astype(np.float64)
        b = rng.uniform(2, 40, N).astype(np.float32).astype(np.float64)
        c = rng.uniform(0.5, 2, N).astype(np.float32).astype(np.float64)
    pg = [rng.permutation(LAT) for _ in range(N)]
    pu = [rng.permutation(LAT) for _ in range(N)]
    pd = [rng.permutation(LAT) for _ in range(N)]
    tau = rng.permutation(D)[:LAT]
    q1, q2, q3 = rng.permutation(S), rng.permutation(S), rng.permutation(D)
    gs, us, vs = 1.75, 9.0, 0.625
    gamma = rng.uniform(0.5, 1.5, LAT).astype(np.float32).astype(np.float64)
    inp = dict(
        x=x, w_router=np.zeros((N, D)), logit_offset=LOGIT_OFFSET.copy(),
        w_down=_perm_matrix(LAT, D, sigma),
        w_gate=np.stack([a[e] * _perm_matrix(LAT, LAT, pg[e]) for e in range(N)]),
        w_uproj=np.stack([b[e] * _perm_matrix(LAT, LAT, pu[e]) for e in range(N)]),
        w_dn=np.stack([c[e] * _perm_matrix(LAT, LAT, pd[e]) for e in range(N)]),
        rms_gamma=gamma,
        w_up=_perm_matrix(LAT, D, tau).T.copy(),
        ws_gate=gs * _perm_matrix(S, D, q1), ws_up=us * _perm_matrix(S, D, q2),
        ws_down=vs * _perm_matrix(D, S, q3),
    )
    par = dict(sigma=sigma, a=a, b=b, c=c, pg=pg, pu=pu, pd=pd, tau=tau, q=(q1, q2, q3),
               shared=(gs, us, vs), gamma=gamma)
    return inp, par


def situ(g, u):
    """SiLU(4 tanh(g/4)) * 25 tanh(u/25)."""
    gc = 4.0 * np.tanh(g / 4.0)
    return gc / (1.0 + np.exp(-gc)) * 25.0 * np.tanh(u / 25.0)


def expected(inp, par, idx, w, act=lambda v: v):
    """The layer output by hand for routing (idx, w); ``act`` is applied to
    every expert input z and every SiTU-GLU output h (identity by default)."""
    x = inp["x"]
    q1, q2, q3 = par["q"]
    gs, us, vs = par["shared"]
    a, b, c = par["a"], par["b"], par["c"]
    out = np.zeros((x.shape[0], D))
    for t in range(x.shape[0]):
        z = act(x[t, par["sigma"]])
        y = np.zeros(LAT)
        for j, e in enumerate(idx[t]):
            h = act(situ(a[e] * z[par["pg"][e]], b[e] * z[par["pu"][e]]))
            y += w[t, j] * c[e] * h[par["pd"][e]]
        yhat = y / np.sqrt(np.mean(y * y) + EPS) * par["gamma"]
        out[t, par["tau"]] += yhat
        out[t] += vs * situ(gs * x[t, q1], us * x[t, q2])[q3]
    return out
