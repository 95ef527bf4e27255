#!/usr/bin/env python3
"""Stable LatentMoE layer throughput on one MI355X.

One step = one moe_latent_forward call over a batch already resident in HBM:
router, Quantile Balancing on the batch, permutation, latent down-projection,
shared gate/up, routed gate/up with SiTU-GLU, routed down, combine + RMSNorm,
up-projection fused with the shared down-projection.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload k3_prefill]

Prints one JSON line.  ``roofline`` describes the dominant kernel (the routed
gate/up grouped GEMM), whose duration is measured with HIP events recorded by
the library around that launch on its stream; ``cpu_baseline`` times the
float64 oracle on a bounded sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0   # dense fp8 MFMA (the W4A8 experts' E4M3 x E2M1 products)
PEAK_FP4_TFLOPS = 10100.0  # dense fp4 MFMA (the W4A4 experts' E2M1 x E2M1 products)
# HBM bytes per launch of the dominant kernel (the routed gate/up launch of a
# layer, the routing loop of the qb workload), from rocprofv3 FETCH_SIZE and
# WRITE_SIZE runs scaled by a 1 GiB device copy (profiles/layer_<workload>.txt,
# profiles/routing_qb_57344x896.txt); None where not measured for the current
# kernel.  Keyed by (workload, qb mode).
TRAFFIC = {("k3_prefill", "batch"): 27.006e9,      # gemm_pipe<96, 256, 1, 3, 64, 3, true, 4, false>
           ("k3_decode", "batch"): 26.313e9,       # gemm_pipe<32, 256, 1, 3, 64, 3, true, 4, false>
           ("k3_prefill_16k", "batch"): 29.231e9,  # gemm_pipe<320, 256, 2, 3, 64, 2, true, 8, false>
           ("k3_mxfp4", "batch"): 9.928e9,         # gemm_pipe_fp4<320, 256, 2, 3, 8, true, 0, 3>
           ("k3_mxfp4", "frozen"): 12.680e9,       # the same kernel, skewed loads (several tiles per expert)
           ("k3_mxfp4_a8", "batch"): 9.111e9,      # gemm_pipe_fp4<320, 256, 2, 3, 8, true, 8, 2>
           ("k3_mxfp4_a4", "batch"): 8.592e9,      # gemm_pipe_fp4<320, 256, 2, 3, 8, true, 4, 3>
           ("tiny", "batch"): 2.369e6,             # gemm_f32<EPI_SITU>
           ("qb", "batch"): 20.967e9}              # route_loop<14>
METRIC = "Stable LatentMoE layer tokens/s on 1 MI355X; MFMA util & HBM GB/s vs peak"


def layer_flops_per_token(s):
    """Matmul flops per token (routed experts counted k times)."""
    dense = 2 * s.d * s.latent * 2 + 2 * s.d * s.shared * 3
    routed = s.k * (2 * s.latent * s.m * 3)
    router = 2 * s.d * s.n
    return dense + routed, router


def weight_bytes(s, touched):
    eb = 2 if s.act == "bf16" else 4
    if s.routed in ("mxfp4", "mxfp4_a8", "mxfp4_a4"):
        per_expert = 3 * s.m * s.latent // 2 + 3 * s.m * s.latent // 32
    else:
        per_expert = 3 * s.m * s.latent * eb
    dense = (2 * s.d * s.latent + 3 * s.d * s.shared) * eb + s.n * s.d * 4
    return touched * per_expert, dense


def gate_up_bytes(s, touched, T):
    """Algorithmic HBM bytes of one routed gate/up launch: the gate and up
    weights of every expert that received a token, the latent rows z read
    once (a token's row serves all k of its experts) and the SiTU-GLU output
    written (one row per token and chosen expert)."""
    eb = 2 if s.act == "bf16" else 4
    if s.routed in ("mxfp4", "mxfp4_a8", "mxfp4_a4"):
        w = touched * 2 * (s.m * s.latent // 2 + s.m * s.latent // 32)
    else:
        w = touched * 2 * s.m * s.latent * eb
    if s.routed == "mxfp4_a8":  # E4M3 codes and E8M0 scales of z
        return w + T * (s.latent + s.latent // 32) + T * s.k * s.m * eb
    if s.routed == "mxfp4_a4":  # E2M1 codes (two per byte) and E8M0 scales of z
        return w + T * (s.latent // 2 + s.latent // 32) + T * s.k * s.m * eb
    return w + T * s.latent * eb + T * s.k * s.m * eb


def cpu_baseline(inp, shape, sample_tokens):
    """The oracle as it stands, on the host: routing of the whole batch (router
    + QB) and the layer for ``sample_tokens`` tokens; per-token time scaled."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    from oracle import layer as olayer
    from oracle import qb

    x = inp["x"].float().cpu()
    host = {"x": x, "w_router": inp["w_router"].cpu(),
            "logit_offset": None if inp["logit_offset"] is None else inp["logit_offset"].cpu()}
    t0 = time.perf_counter()
    s = olayer.router_scores(olayer.as_f64(host["x"]), olayer.as_f64(host["w_router"]),
                             None if host["logit_offset"] is None
                             else olayer.as_f64(host["logit_offset"]))
    r = qb.route_qb(s, shape.k)
    t_route = time.perf_counter() - t0
    tokens = np.arange(sample_tokens)
    need = np.unique(r["idx"][tokens])
    # copy only the experts the sample needs to the host (not timed)
    def subset(w):
        if isinstance(w, tuple):
            return tuple({int(e): w[i][int(e)].cpu() for e in need} for i in range(2))
        return {int(e): w[int(e)].cpu() for e in need}
    lay = dict(x=x, w_down=inp["w_down"].cpu(), w_up=inp["w_up"].cpu(),
               w_gate=subset(inp["w_gate"]), w_uproj=subset(inp["w_uproj"]),
               w_dn=subset(inp["w_dn"]), rms_gamma=inp["rms_gamma"].cpu(),
               ws_gate=inp["ws_gate"].cpu(), ws_up=inp["ws_up"].cpu(),
               ws_down=inp["ws_down"].cpu())
    t1 = time.perf_counter()
    olayer.layer_forward(lay, r["idx"], r["w"], shape.eps, tokens=tokens,
                         act_mxfp8=shape.routed == "mxfp4_a8",
                         act_mxfp4=shape.routed == "mxfp4_a4")
    t_layer = time.perf_counter() - t1
    per_token = t_route / shape.T + t_layer / sample_tokens
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": 1.0 / per_token, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "logical_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": (f"oracle router + QB on the full batch of {shape.T} tokens "
                       f"({t_route:.1f} s) and the float64 layer on {sample_tokens} tokens "
                       f"({t_layer:.1f} s); tokens/s = 1 / (route_s/T + layer_s/sample)")}


def time_backward(moe, sh, w, x, bias0, ws, shape, args):
    """moe_latent_backward on this batch's routing (from one forward call) and
    a seeded N(0,1) output gradient: ms per call, timed like the forward."""
    import torch
    fwd = moe.latent_forward(sh, w, x, bias=bias0, workspace=ws, want_scores=True)
    g = torch.Generator(device=x.device)
    g.manual_seed(1234)
    dout = torch.randn(x.shape, generator=g, device=x.device, dtype=torch.float32).to(x.dtype)
    bws = torch.empty(moe.lib().moe_backward_workspace_bytes(ctypes_ref(sh)), dtype=torch.uint8,
                      device=x.device)

    def step():
        return moe.latent_backward(sh, w, x, fwd["scores"], fwd["idx"], fwd["w"], dout,
                                   workspace=bws)

    r = step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        r = step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    del r, bws
    torch.cuda.empty_cache()
    return {"ms_per_step": ms, "tokens_per_s": shape.T / (ms / 1e3),
            "what": "gradients of x and every weight for one forward call (forward activations "
                    "recomputed inside), selection held fixed"}


def time_train(moe, sh, w, x, bias0, ws, shape, args, mode="saved"):
    """One training step: forward with QB on the batch (the bias carried from
    step to step), backward with a seeded N(0,1) output gradient, and the SGD
    update of every weight in place (lr 1e-6).  mode "saved": the training
    forward keeps its activations and the backward reads them, the update
    fused into the experts' weight-gradient GEMMs; "fused": the backward
    recomputes the activations, update fused; "separate": moe_latent_backward,
    then moe_sgd_step.  Timed like the forward; the weights change from step
    to step as in training."""
    import torch
    g = torch.Generator(device=x.device)
    g.manual_seed(4321)
    dout = torch.randn(x.shape, generator=g, device=x.device, dtype=torch.float32).to(x.dtype)
    bws = torch.empty(moe.lib().moe_backward_workspace_bytes(ctypes_ref(sh)), dtype=torch.uint8,
                      device=x.device)
    bias = bias0.clone()
    saved = (torch.empty(moe.saved_activations_bytes(sh), dtype=torch.uint8, device=x.device)
             if mode == "saved" else None)

    def step():
        nonlocal bias
        fwd = moe.latent_forward(sh, w, x, bias=bias, workspace=ws, want_scores=True, saved=saved)
        bias = fwd["bias"]
        if mode == "saved":
            moe.latent_backward_train(sh, w, x, fwd["scores"], fwd["idx"], fwd["w"], dout, saved,
                                      lr=1e-6, workspace=bws)
        elif mode == "fused":
            moe.latent_backward_sgd(sh, w, x, fwd["scores"], fwd["idx"], fwd["w"], dout, 1e-6,
                                    workspace=bws)
        else:
            grads = moe.latent_backward(sh, w, x, fwd["scores"], fwd["idx"], fwd["w"], dout,
                                        workspace=bws)
            moe.sgd_step(sh, w, grads, 1e-6)

    step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    del bws, saved
    torch.cuda.empty_cache()
    return {"ms_per_step": ms, "tokens_per_s": shape.T / (ms / 1e3),
            "what": "forward (QB on the batch) + backward + SGD update of every weight" + {
                "saved": " (activations kept by the forward; update fused into the expert "
                         "weight-gradient GEMMs)",
                "fused": " (activations recomputed; update fused)",
                "separate": " (activations recomputed; backward and update as two calls)"}[mode]}


def time_graph(step, shape, args):
    """The timed forward step captured once in a HIP graph and replayed
    (same inputs, same kernels; no host launch work per step)."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    del g
    return {"ms_per_step": ms, "tokens_per_s": shape.T / (ms / 1e3),
            "what": "the same forward step captured once in a HIP graph and replayed"}


def ctypes_ref(obj):
    import ctypes
    return ctypes.byref(obj)


def sign_baseline(moe, sh, w, x, bias0, ws, shape):
    """QB and the fixed-step sign update on the router scores of this batch:
    updates made, status, max |load - target| and the routing time."""
    import torch
    scores = moe.latent_forward(sh, w, x, bias=bias0, workspace=ws, want_scores=True)["scores"]
    scores = scores.contiguous()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ev[0].record()
        r = fn()
        ev[1].record()
        torch.cuda.synchronize()
        return r, ev[0].elapsed_time(ev[1])

    r, ms = timed(lambda: moe.route_qb(scores, shape.k))
    info = [int(v) for v in r["info"].cpu()]
    out = {"scores": "this batch's router scores",
           "qb": {"rounds": info[0], "moves": info[3], "status": info[1],
                  "max_abs_imbalance": info[2], "ms": ms}}
    rows = []
    for step in (2.0 ** -7, 2.0 ** -10, 2.0 ** -13):
        for rounds in (64, 256, 1024):
            r, ms = timed(lambda: moe.route_sign(scores, shape.k, step, rounds))
            info = [int(v) for v in r["info"].cpu()]
            rows.append({"step": step, "max_rounds": rounds, "updates": info[0],
                         "status": info[1], "max_abs_imbalance": info[2], "ms": ms})
    out["sign"] = rows
    return out


QB_METRIC = "Quantile Balancing routing tokens/s on 1 MI355X; HBM GB/s vs peak"


def qb_scores(T, n, offset_std, seed):
    """Sigmoid scores (fp32) of the routing-only workload's seeded logits."""
    import numpy as np

    import workloads
    z = workloads.qb_logits(T, n, offset_std, seed).astype(np.float64)
    return (1.0 / (1.0 + np.exp(-z))).astype(np.float32)


def qb_cpu_baseline(cfg, sample_tokens):
    """The oracle's routing (Quantile Balancing on the host, float64 keys) on a
    batch of ``sample_tokens`` tokens of the same distribution."""
    from threadpoolctl import threadpool_info

    from oracle import qb
    s = qb_scores(sample_tokens, cfg["n"], cfg["offset_std"], seed=1)
    t0 = time.perf_counter()
    r = qb.route_qb(s, cfg["k"])
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle", "logical_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "sample": (f"oracle route_qb on {sample_tokens} tokens x {cfg['n']} experts, "
                       f"k={cfg['k']} ({dt:.1f} s, {r['info'][0]} rounds + "
                       f"{r['info'][3]} moves)")}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_reference(nbytes, dev):
    """One plain device-to-device copy of nbytes: the reference that scales
    FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def run_qb(args):
    """Routing-only workload: Quantile Balancing of T=57344 tokens over n=896
    experts, k=16, scores from N(0,1) logits plus a per-expert N(0, 0.5^2)
    offset.  One step = one moe_route_qb call (bias from zero)."""
    import torch

    import sparse_moe_ffn_sigmoid_amd as moe
    import workloads

    cfg = workloads.QB_SHAPE
    T, n, k = cfg["T"], cfg["n"], cfg["k"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    scores = torch.from_numpy(qb_scores(T, n, cfg["offset_std"], seed=0)).to(dev)
    ws = torch.empty(max(moe.route_workspace_bytes(T, n, k), 256), dtype=torch.uint8, device=dev)

    def step():
        return moe.route_qb(scores, k, workspace=ws)

    for _ in range(args.warmup):
        r = step()
    torch.cuda.synchronize()
    moe.stage_timing(True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        r = step()
    end.record()
    torch.cuda.synchronize()
    stages = moe.stage_times()
    moe.stage_timing(False)
    ms_per_step = start.elapsed_time(end) / args.steps
    info = [int(v) for v in r["info"].cpu()]
    r_ms, r_n = stages["routing"]
    avg_ms = r_ms / max(r_n, 1)
    # one read of the fp32 scores per quantile round or augmenting-path move,
    # one for the final pass, and the idx / w outputs
    passes = info[0] + info[3] + 1
    algo = passes * 4.0 * T * n + 8.0 * T * k
    roof = {"bound": "hbm", "achieved": algo / (avg_ms / 1e3) / 1e9, "peak": PEAK_HBM_GBS,
            "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = TRAFFIC.get(("qb", "batch"))
    rec = {
        "metric": QB_METRIC, "value": T / (ms_per_step / 1e3), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0,1) logits + per-expert N(0,0.25) offsets, fp32 sigmoid)",
        "config": {"workload": "qb_routing_57344x896", "T": T, "experts": n, "top_k": k,
                   "offset_std": cfg["offset_std"], "qb": "batch"},
        "roofline": dict(roof, kernel="routing loop (one persistent launch per call)",
                         bytes_per_launch=algo, avg_ms=avg_ms, passes=passes),
        "qb_info": info,
    }
    if args.copy_bytes > 0:
        copy_reference(args.copy_bytes, dev)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = qb_cpu_baseline(cfg, args.cpu_sample_qb_tokens)
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="k3_prefill",
                    choices=["k3_prefill", "k3_decode", "k3_mxfp4", "k3_mxfp4_a8", "k3_mxfp4_a4",
                             "k3_prefill_16k",
                             "tiny", "qb"])
    ap.add_argument("--qb", default="batch", choices=["batch", "frozen"])
    ap.add_argument("--cpu-sample-tokens", type=int, default=2)
    ap.add_argument("--cpu-sample-qb-tokens", type=int, default=8192,
                    help="tokens of the routing-only oracle sample (--workload qb)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sign-baseline", action="store_true",
                    help="also route this batch's scores with the fixed-step sign update "
                         "(DeepSeek-V3's bias rule) and report rounds / imbalance / time beside QB")
    ap.add_argument("--graph", action="store_true",
                    help="also time the forward step captured in a HIP graph and replayed; "
                         "reported under 'graph'")
    ap.add_argument("--train", action="store_true",
                    help="also time a training step (forward, backward, SGD update; bf16 layers); "
                         "reported under 'train', after every other measurement (it changes "
                         "the weights)")
    ap.add_argument("--backward", action="store_true",
                    help="also time moe_latent_backward (bf16 layers) on this batch's routing and "
                         "a random output gradient; reported under 'backward'")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="after the run, one plain device-to-device copy of this many bytes "
                         "(the reference for scaling FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one MI355X: the layer here runs on a single GPU "
              "(no sharding or collectives); use --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.workload == "qb":
        run_qb(args)
        return

    import torch

    import sparse_moe_ffn_sigmoid_amd as moe
    import workloads

    shape = workloads.SHAPES[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = workloads.layer_inputs(shape, dev, seed=0)
    w = {}
    for key, v in inp.items():
        if key == "x" or v is None:
            continue
        if isinstance(v, tuple):
            w[key] = v[0]
            w[{"w_gate": "s_gate", "w_uproj": "s_uproj", "w_dn": "s_dn"}[key]] = v[1]
        else:
            w[key] = v
    if "logit_offset" in w:
        w["router_logit_offset"] = w.pop("logit_offset")
    act = {"f32": moe.MOE_F32, "bf16": moe.MOE_BF16}[shape.act]
    routed = {"f32": moe.MOE_F32, "bf16": moe.MOE_BF16, "mxfp4": moe.MOE_MXFP4,
              "mxfp4_a8": moe.MOE_MXFP4_A8, "mxfp4_a4": moe.MOE_MXFP4_A4}[shape.routed]
    qb_mode = moe.MOE_QB_BATCH if args.qb == "batch" else moe.MOE_QB_FROZEN
    sh = moe.make_shape(shape.T, shape.d, shape.latent, shape.n, shape.k, shape.m, shape.shared,
                        act, routed, shape.eps, qb_mode, 64)
    ws = torch.empty(moe.forward_workspace_bytes(sh), dtype=torch.uint8, device=dev)
    bias0 = torch.zeros(shape.n, dtype=torch.float64, device=dev)
    x = inp["x"]

    def step():
        return moe.latent_forward(sh, w, x, bias=bias0, workspace=ws)

    for _ in range(args.warmup):
        r = step()
    torch.cuda.synchronize()
    moe.stage_timing(True)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        r = step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stages = moe.stage_times()
    moe.stage_timing(False)
    ms_per_step = start.elapsed_time(end) / args.steps
    tokens_per_s = shape.T / (ms_per_step / 1e3)

    loads = r["loads"].cpu()
    touched = int((loads > 0).sum())
    info = [int(v) for v in r["info"].cpu()]
    flops, router_flops = layer_flops_per_token(shape)
    wb_routed, wb_dense = weight_bytes(shape, touched)
    gu_ms, gu_n = stages["routed_gate_up"]
    gu_avg_ms = gu_ms / max(gu_n, 1)
    gu_bytes = gate_up_bytes(shape, touched, shape.T)
    gu_flops = 2.0 * shape.T * shape.k * (2 * shape.m) * shape.latent
    if shape.routed == "mxfp4_a8":
        # E4M3 x E2M1 on the scaled MFMA: priced at the fp8 MFMA peak
        roof = {"bound": "mfma", "achieved": gu_flops / (gu_avg_ms / 1e3) / 1e12,
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s"}
    elif shape.routed == "mxfp4_a4":
        # E2M1 x E2M1 on the scaled MFMA: priced at the fp4 MFMA peak
        roof = {"bound": "mfma", "achieved": gu_flops / (gu_avg_ms / 1e3) / 1e12,
                "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s"}
    elif shape.routed == "mxfp4" or shape.T * shape.k >= 32 * shape.n * 8:
        # codes decoded to bf16, or hundreds of rows per expert: compute-bound,
        # bf16 dense MFMA peak
        roof = {"bound": "mfma", "achieved": gu_flops / (gu_avg_ms / 1e3) / 1e12,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": gu_bytes / (gu_avg_ms / 1e3) / 1e9,
                "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = TRAFFIC.get((args.workload, args.qb))
    rec = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16; routed experts mxfp8 x mxfp4" if shape.routed == "mxfp4_a8"
                  else "bf16; routed experts mxfp4 x mxfp4" if shape.routed == "mxfp4_a4"
                  else "bf16" if shape.act == "bf16" else "f32"),
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights, skewed router offsets)",
        "config": {"workload": {"k3_prefill": "k3_prefill_bf16", "k3_decode": "k3_decode_bf16",
                                "k3_mxfp4": "k3_prefill_mxfp4",
                                "k3_mxfp4_a8": "k3_prefill_mxfp4_w4a8",
                                "k3_mxfp4_a4": "k3_prefill_mxfp4_w4a4",
                                "k3_prefill_16k": "k3_prefill_bf16_16k",
                                "tiny": "tiny_fp32_latency"}[args.workload],
                   "T": shape.T, "d": shape.d, "latent": shape.latent, "experts": shape.n,
                   "top_k": shape.k, "inter": shape.m, "shared_inter": shape.shared,
                   "routed_weights": shape.routed, "qb": args.qb},
        "roofline": dict(roof, kernel="routed gate/up grouped GEMM + SiTU-GLU",
                         bytes_per_launch=gu_bytes, flops_per_launch=gu_flops, avg_ms=gu_avg_ms),
        "layer": {
            "hbm_gbs": (wb_routed + wb_dense) / (ms_per_step / 1e3) / 1e9,
            "weight_bytes": wb_routed + wb_dense,
            "mfma_util": (flops + router_flops) * shape.T / (ms_per_step / 1e3) / (PEAK_BF16_TFLOPS * 1e12),
            "experts_touched": touched,
            "qb_info": info,
            "stages_ms": {k: v[0] / max(v[1], 1) for k, v in stages.items()},
            "wall_s": wall,
        },
    }
    if args.sign_baseline:
        rec["routing_baseline"] = sign_baseline(moe, sh, w, x, bias0, ws, shape)
    if args.backward:
        rec["backward"] = time_backward(moe, sh, w, x, bias0, ws, shape, args)
    if args.graph:
        rec["graph"] = time_graph(step, shape, args)
    if args.copy_bytes > 0:
        copy_reference(args.copy_bytes, dev)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(inp, shape, args.cpu_sample_tokens)
    if args.train:  # last: it updates the weights in place
        rec["train"] = time_train(moe, sh, w, x, bias0, ws, shape, args)
        rec["train_recompute"] = time_train(moe, sh, w, x, bias0, ws, shape, args, mode="fused")
        rec["train_separate"] = time_train(moe, sh, w, x, bias0, ws, shape, args,
                                           mode="separate")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
