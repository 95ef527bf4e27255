"""moe_latent_forward and moe_route_qb captured in a HIP graph.

Every launch of a call goes onto the caller's stream (the shared branch forks
onto the library's side stream and joins back through events), so a call can
be captured.  Each replay must give bit-identical outputs to the eager call
on the same inputs, with other eager work and synchronisations between the
replays.
"""
import numpy as np
import pytest
import torch

import workloads
from layer_cases import announce, make_shape, to_device

pytestmark = pytest.mark.gpu

FIELDS = ("out", "idx", "w", "loads", "bias", "info")


def host(r):
    return {k: (v.view(torch.int16) if v.dtype == torch.bfloat16 else v).cpu().numpy()
            for k, v in r.items() if v is not None}


def assert_same(a, b, what):
    for k in a:
        assert a[k].dtype == b[k].dtype and np.array_equal(a[k], b[k]), f"{what}: {k} differs"


@pytest.mark.parametrize("routed,qb_mode", [("bf16", 1), ("mxfp4_a8", 1), ("mxfp4", 0)])
def test_layer_graph_replays_bit_identical(routed, qb_mode):
    import sparse_moe_ffn_sigmoid_amd as moe
    kw = dict(T=300, n=16, k=4, d=1024, latent=512, m=512, shared=256) if routed != "bf16" \
        else dict(T=200)
    shape = workloads.small_shape(routed=routed, **kw)
    announce(f"graph layer {routed} qb_mode={qb_mode}")
    inp = workloads.layer_inputs(shape, "cpu", seed=3)
    x, w = to_device(inp)
    w["router_logit_offset"] = w.pop("logit_offset")
    x2 = torch.flip(x, dims=[0]).contiguous()
    sh = make_shape(moe, shape, qb_mode=qb_mode)
    ws = torch.empty(moe.forward_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    bias = torch.linspace(-0.01, 0.01, shape.n, dtype=torch.float64, device="cuda")

    def fwd(inp_x):
        return moe.latent_forward(sh, w, inp_x, bias=bias, workspace=ws)

    eager = host(fwd(x))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd(x)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r_g = fwd(x)
    torch.cuda.synchronize()
    for rep in range(3):
        other = host(fwd(x2))  # eager work between the replays, same workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(eager, host(r_g), f"replay {rep}")
        assert not np.array_equal(other["idx"], eager["idx"])


def test_route_graph_replays_bit_identical():
    import sparse_moe_ffn_sigmoid_amd as moe
    announce("graph route_qb T=4096 n=896 k=16")
    T, n, k = 4096, 896, 16
    z = workloads.qb_logits(T, n, 0.5, seed=5).astype(np.float64)
    s = torch.from_numpy((1.0 / (1.0 + np.exp(-z))).astype(np.float32)).cuda()
    ws = torch.empty(moe.route_workspace_bytes(T, n, k), dtype=torch.uint8, device="cuda")
    eager = host(moe.route_qb(s, k, workspace=ws))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.route_qb(s, k, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        r_g = moe.route_qb(s, k, workspace=ws)
    torch.cuda.synchronize()
    s2 = torch.flip(s, dims=[1]).contiguous()
    for rep in range(3):
        moe.route_qb(s2, k, workspace=ws)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(eager, host(r_g), f"replay {rep}")


def test_training_step_graph_replays_match_eager_steps():
    """One training step (training forward with QB on the batch, the bias
    carried in a device buffer, then the backward with the fused SGD update
    reading the saved activations) captured once: three replays from the
    initial weights give the outputs and the weights of three eager steps,
    bit for bit."""
    import sparse_moe_ffn_sigmoid_amd as moe
    shape = workloads.small_shape(T=200)
    announce("graph training step")
    inp = workloads.layer_inputs(shape, "cpu", seed=12, random_gamma=True)
    x, w0 = to_device(inp)
    w0["router_logit_offset"] = w0.pop("logit_offset")
    sh = make_shape(moe, shape)
    ws = torch.empty(moe.forward_workspace_bytes(sh), dtype=torch.uint8, device="cuda")
    bws = torch.empty(moe.lib().moe_backward_workspace_bytes(ctypes_ref(moe, sh)),
                      dtype=torch.uint8, device="cuda")
    saved = torch.empty(moe.saved_activations_bytes(sh), dtype=torch.uint8, device="cuda")
    dout = torch.randn((shape.T, shape.d), generator=torch.Generator().manual_seed(4)).to(
        torch.bfloat16).cuda()
    bias = torch.zeros(shape.n, dtype=torch.float64, device="cuda")

    def step(wd):
        f = moe.latent_forward(sh, wd, x, bias=bias, workspace=ws, want_scores=True, saved=saved)
        bias.copy_(f["bias"])
        moe.latent_backward_train(sh, wd, x, f["scores"], f["idx"], f["w"], dout, saved, lr=1e-3,
                                  workspace=bws)
        return f["out"]

    w_e = {k: v.clone() for k, v in w0.items()}
    outs = []
    for _ in range(3):
        outs.append(step(w_e).view(torch.int16).cpu().numpy())
    torch.cuda.synchronize()
    w_g = {k: v.clone() for k, v in w0.items()}
    bias.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out_g = step(w_g)
    torch.cuda.synchronize()
    for i in range(3):
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out_g.view(torch.int16).cpu().numpy(), outs[i]), f"replay {i}"
        torch.zeros(1 << 20, device="cuda").sum()  # other eager work between the replays
    for k in w_e:
        a, b = w_e[k], w_g[k]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), k
    del g


def ctypes_ref(moe, sh):
    import ctypes
    return ctypes.byref(sh)
