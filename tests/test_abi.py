"""The C ABI library loads, exports every declared entry point and validates
arguments on the host before launching anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ("moe_route_qb", "moe_latent_forward", "moe_route_workspace_bytes",
                 "moe_forward_workspace_bytes", "moe_status_str"):
        assert want in names


def test_library_exports_every_declared_symbol():
    import sparse_moe_ffn_sigmoid_amd as moe
    lib = ctypes.CDLL(moe.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(moe.EXPORTED) <= set(declared_functions())


def test_status_strings():
    import sparse_moe_ffn_sigmoid_amd as moe
    lib = moe.lib()
    assert lib.moe_status_str(0) == b"ok"
    assert b"workspace" in lib.moe_status_str(-3)
    assert lib.moe_status_str(12345)


def test_route_validation_on_host():
    import sparse_moe_ffn_sigmoid_amd as moe
    lib = moe.lib()
    fake = ctypes.c_void_p(1 << 20)            # never dereferenced: validation fails first
    assert lib.moe_route_workspace_bytes(100, 0, 1) == 0
    assert lib.moe_route_workspace_bytes(100, 8, 9) == 0
    assert lib.moe_route_workspace_bytes(100, 2048, 4) == 0
    need = lib.moe_route_workspace_bytes(100, 64, 4)
    assert need > 0
    args = lambda T, n, k, mode=1, ws=fake, wsb=need: (fake, T, n, k, mode, 64, fake, fake, fake,
                                                       fake, fake, ws, wsb, None)
    assert lib.moe_route_qb(*args(100, 64, 65)) == -1          # k > n
    assert lib.moe_route_qb(*args(100, 64, 0)) == -1
    assert lib.moe_route_qb(*args(-1, 64, 4)) == -1
    assert lib.moe_route_qb(*args(100, 2048, 4)) == -2         # n > 1024
    assert lib.moe_route_qb(*args(100, 128, 100)) == -2        # k > 64
    assert lib.moe_route_qb(*args(100, 64, 4, mode=7)) == -1
    assert lib.moe_route_qb(*args(100, 64, 4, ws=None)) == -1
    assert lib.moe_route_qb(*args(100, 64, 4, ws=ctypes.c_void_p((1 << 20) + 8))) == -1
    assert lib.moe_route_qb(*args(100, 64, 4, wsb=need - 1)) == -3


def test_route_noalloc_validation_on_host():
    import sparse_moe_ffn_sigmoid_amd as moe
    lib = moe.lib()
    fake = ctypes.c_void_p(1 << 20)            # never dereferenced: validation fails first
    args = lambda T, n, k, mode=1: (fake, T, n, k, mode, 64, fake, fake, fake, fake, fake, None)
    assert lib.moe_route_qb_noalloc(*args(100, 64, 65)) == -1          # k > n
    assert lib.moe_route_qb_noalloc(*args(100, 2048, 4)) == -2         # n > 1024
    assert lib.moe_route_qb_noalloc(*args(100, 64, 4, mode=7)) == -1
    assert lib.moe_route_qb_noalloc(*args(8192, 896, 16)) == -3        # beyond the scratch array
    assert lib.moe_route_workspace_bytes(6000, 896, 16) <= 32 << 20    # the K3 decode / prefill sizes fit


def test_backward_validation_on_host():
    import sparse_moe_ffn_sigmoid_amd as moe
    lib = moe.lib()
    ws = lambda **kw: lib.moe_backward_workspace_bytes(ctypes.byref(_shape(moe, **kw)))
    assert ws() > 0 and ws(T=0) > 0
    assert ws(routed=moe.MOE_MXFP4) == 0                      # bf16 layers only
    assert ws(act=moe.MOE_F32, routed=moe.MOE_F32) == 0
    assert ws(k=897) == 0 and ws(d=7168 + 32) == 0
    fake = ctypes.c_void_p(1 << 20)            # never dereferenced: validation fails first
    sh = _shape(moe, T=64)
    wts = moe.MoeWeights(*([1 << 20] * len(moe.MoeWeights._fields_)))
    grads = moe.MoeGrads(*([1 << 20] * len(moe.MoeGrads._fields_)))
    need = ws(T=64)
    call = lambda g=grads, w=wts, ws_=fake, nbytes=need: lib.moe_latent_backward(
        ctypes.byref(sh), ctypes.byref(w), fake, fake, fake, fake, fake, ctypes.byref(g), ws_,
        nbytes, None)
    assert call(nbytes=need - 1) == -3
    assert call(ws_=ctypes.c_void_p((1 << 20) + 8)) == -1
    no_off = moe.MoeGrads(*([1 << 20] * len(moe.MoeGrads._fields_)))
    no_off.d_router_logit_offset = None                    # the weights have an offset
    assert call(g=no_off) == -1
    no_dx = moe.MoeGrads(*([1 << 20] * len(moe.MoeGrads._fields_)))
    no_dx.dx = None
    assert call(g=no_dx) == -1


def test_mxfp4_quantize_validation_on_host():
    import sparse_moe_ffn_sigmoid_amd as moe
    lib = moe.lib()
    fake = ctypes.c_void_p(1 << 20)            # never dereferenced: validation fails first
    assert lib.moe_mxfp4_quantize(fake, 4, 48, fake, fake, None) == -1       # K % 32
    assert lib.moe_mxfp4_quantize(fake, -1, 64, fake, fake, None) == -1
    assert lib.moe_mxfp4_quantize(None, 4, 64, fake, fake, None) == -1
    assert lib.moe_mxfp4_quantize(ctypes.c_void_p((1 << 20) + 8), 4, 64, fake, fake, None) == -1
    assert lib.moe_mxfp4_quantize(fake, 4, 64, ctypes.c_void_p((1 << 20) + 2), fake, None) == -1
    assert lib.moe_mxfp4_quantize(None, 0, 64, None, None, None) == 0


def test_mxfp8_quantize_validation_on_host():
    import sparse_moe_ffn_sigmoid_amd as moe
    lib = moe.lib()
    fake = ctypes.c_void_p(1 << 20)            # never dereferenced: validation fails first
    assert lib.moe_mxfp8_quantize(fake, 4, 48, fake, fake, None) == -1       # K % 32
    assert lib.moe_mxfp8_quantize(fake, 4, 0, fake, fake, None) == -1
    assert lib.moe_mxfp8_quantize(fake, -1, 64, fake, fake, None) == -1
    assert lib.moe_mxfp8_quantize(None, 4, 64, fake, fake, None) == -1
    assert lib.moe_mxfp8_quantize(fake, 4, 64, fake, None, None) == -1
    assert lib.moe_mxfp8_quantize(ctypes.c_void_p((1 << 20) + 2), 4, 64, fake, fake, None) == -1
    assert lib.moe_mxfp8_quantize(fake, 4, 64, ctypes.c_void_p((1 << 20) + 4), fake, None) == -1
    assert lib.moe_mxfp8_quantize(None, 0, 64, None, None, None) == 0       # nothing to do


def test_binding_fails_loudly_without_library(tmp_path):
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "sparse_moe_ffn_sigmoid_amd")
    dst = tmp_path / "sparse_moe_ffn_sigmoid_amd"
    dst.mkdir()
    (dst / "__init__.py").write_text(open(os.path.join(pkg, "__init__.py")).read())
    r = subprocess.run([sys.executable, "-c", "import sparse_moe_ffn_sigmoid_amd"],
                       cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode != 0 and "libmoe_mi355x.so is missing" in r.stderr


def test_sign_route_validation_on_host():
    import sparse_moe_ffn_sigmoid_amd as moe
    lib = moe.lib()
    fake = ctypes.c_void_p(1 << 20)            # never dereferenced: validation fails first
    need = lib.moe_route_workspace_bytes(100, 64, 4)
    args = lambda T, n, k, step=2.0 ** -10, rounds=8, ws=fake: (
        fake, T, n, k, ctypes.c_double(step), rounds, fake, fake, fake, fake, fake, ws, need, None)
    assert lib.moe_route_sign(*args(100, 64, 65)) == -1        # k > n
    assert lib.moe_route_sign(*args(100, 2048, 4)) == -2       # n > 1024
    assert lib.moe_route_sign(*args(100, 64, 4, step=0.0)) == -1
    assert lib.moe_route_sign(*args(100, 64, 4, step=-1.0)) == -1
    assert lib.moe_route_sign(*args(100, 64, 4, step=2.0 ** -45)) == -1   # below one grid unit
    assert lib.moe_route_sign(*args(100, 64, 4, step=2.0 ** 11)) == -1    # beyond the bias range
    assert lib.moe_route_sign(*args(100, 64, 4, rounds=-1)) == -1
    assert lib.moe_route_sign(*args(100, 64, 4, ws=None)) == -1


def _shape(moe, **kw):
    base = dict(T=4096, d=7168, latent=3584, n=896, k=16, m=2048, shared=6144,
                act=moe.MOE_BF16, routed=moe.MOE_BF16, eps=1e-6, mode=moe.MOE_QB_BATCH, rounds=64)
    base.update(kw)
    return moe.MoeShape(base["T"], base["d"], base["latent"], base["n"], base["k"], base["m"],
                        base["shared"], base["act"], base["routed"], base["eps"], base["mode"],
                        base["rounds"])


def test_forward_workspace_sizing_on_host():
    import sparse_moe_ffn_sigmoid_amd as moe
    lib = moe.lib()
    ws = lambda **kw: lib.moe_forward_workspace_bytes(ctypes.byref(_shape(moe, **kw)))
    # the K3 prefill batch: scores, routed rows h (bf16) and y (fp32) dominate
    T, k, n, m, L = 4096, 16, 896, 2048, 3584
    need = ws()
    floor = T * n * 4 + T * k * (m * 2 + L * 4)
    assert floor <= need <= floor + (1 << 30)
    assert ws(T=8192) > need > ws(T=64) > 0
    assert ws(T=0) > 0                               # an empty batch is valid
    assert ws(routed=moe.MOE_MXFP4) > 0
    assert ws(act=moe.MOE_F32, routed=moe.MOE_F32) > 0
    # shapes the library does not take: size 0
    assert ws(d=7168 + 32) == 0                      # widths must be multiples of 64
    assert ws(latent=4096 + 64) == 0                 # latent above 4096
    assert ws(k=n + 1) == 0
    assert ws(n=2048) == 0
    assert ws(act=moe.MOE_F32, routed=moe.MOE_MXFP4) == 0
    assert ws(routed=moe.MOE_MXFP4_A8) > ws(routed=moe.MOE_MXFP4)   # room for the MXFP8 rows
    assert ws(routed=moe.MOE_MXFP4_A8, latent=3584 + 64) == 0       # W4A8 widths: multiples of 128
    assert ws(routed=moe.MOE_MXFP4_A8, m=2048 + 64) == 0
    assert ws(routed=moe.MOE_MXFP4_A8) > ws(routed=moe.MOE_MXFP4_A4) > ws(routed=moe.MOE_MXFP4)
    assert ws(routed=moe.MOE_MXFP4_A4, latent=3584 + 64) == 0       # W4A4: the same limits
    assert ws(routed=moe.MOE_MXFP4_A4, act=moe.MOE_F32) == 0
    assert ws(act=moe.MOE_F32, routed=moe.MOE_BF16) == 0
    assert ws(mode=5) == 0


def test_forward_validation_on_host():
    import sparse_moe_ffn_sigmoid_amd as moe
    lib = moe.lib()
    fake = ctypes.c_void_p(1 << 20)                  # never dereferenced: validation fails first
    names = [f[0] for f in moe.MoeWeights._fields_]
    full = moe.MoeWeights(*[fake] * len(names))
    sh = _shape(moe, T=64, d=256, latent=128, n=32, k=4, m=64, shared=128)
    need = lib.moe_forward_workspace_bytes(ctypes.byref(sh))
    assert need > 0

    def call(shape=sh, weights=full, x=fake, out=fake, bias=fake, ws=fake, wsb=need):
        return lib.moe_latent_forward(ctypes.byref(shape), ctypes.byref(weights), x, out, bias,
                                      None, None, None, None, None, None, ws, wsb, None)

    assert call(wsb=need - 1) == -3                  # workspace too small
    assert call(ws=ctypes.c_void_p((1 << 20) + 64)) == -1   # workspace not 256-byte aligned
    assert call(ws=None) == -1
    assert call(bias=None) == -1
    assert call(x=None) == -1
    assert call(out=None) == -1
    for name in ("w_router", "w_down", "w_up", "w_gate", "w_uproj", "w_dn", "rms_gamma",
                 "ws_gate", "ws_up", "ws_down"):
        w = moe.MoeWeights(*[None if f == name else fake for f in names])
        assert call(weights=w) == -1, name
    # MXFP4 routed weights need their E8M0 scales
    mx = _shape(moe, T=64, d=256, latent=128, n=32, k=4, m=64, shared=128, routed=moe.MOE_MXFP4)
    need_mx = lib.moe_forward_workspace_bytes(ctypes.byref(mx))
    no_scales = moe.MoeWeights(*[None if f in ("s_gate", "s_uproj", "s_dn") else fake
                                 for f in names])
    assert call(shape=mx, weights=no_scales, wsb=need_mx) == -1
    assert call(shape=_shape(moe, T=64, d=250, latent=128, n=32, k=4, m=64, shared=128)) == -2


def test_sgd_validation_on_host():
    import sparse_moe_ffn_sigmoid_amd as moe
    lib = moe.lib()
    sh = _shape(moe, T=64)
    wts = moe.MoeWeights(*([1 << 20] * len(moe.MoeWeights._fields_)))
    grads = moe.MoeGrads(*([1 << 20] * len(moe.MoeGrads._fields_)))
    call = lambda s=sh, w=wts, g=grads, lr=0.1: lib.moe_sgd_step(
        None if s is None else ctypes.byref(s), None if w is None else ctypes.byref(w),
        None if g is None else ctypes.byref(g), ctypes.c_float(lr), None)
    assert call(s=None) == -1 and call(w=None) == -1 and call(g=None) == -1
    assert call(lr=float("nan")) == -1 and call(lr=float("inf")) == -1
    no_off = moe.MoeGrads(*([1 << 20] * len(moe.MoeGrads._fields_)))
    no_off.d_router_logit_offset = None                    # the weights have an offset
    assert call(g=no_off) == -1
    no_gate = moe.MoeWeights(*([1 << 20] * len(moe.MoeWeights._fields_)))
    no_gate.w_gate = None
    assert call(w=no_gate) == -1
    assert call(s=_shape(moe, T=64, routed=moe.MOE_MXFP4)) == -2   # bf16 layers only


def test_fused_backward_sgd_validation_on_host():
    import sparse_moe_ffn_sigmoid_amd as moe
    lib = moe.lib()
    fake = ctypes.c_void_p(1 << 20)            # never dereferenced: validation fails first
    sh = _shape(moe, T=64)
    need = lib.moe_backward_workspace_bytes(ctypes.byref(sh))
    wts = moe.MoeWeights(*([1 << 20] * len(moe.MoeWeights._fields_)))
    grads = moe.MoeGrads(*([1 << 20] * len(moe.MoeGrads._fields_)))
    call = lambda g=grads, lr=0.1, ws_=fake, nbytes=need, s=sh: lib.moe_latent_backward_sgd(
        ctypes.byref(s), ctypes.byref(wts), fake, fake, fake, fake, fake, ctypes.byref(g),
        ctypes.c_float(lr), ws_, nbytes, None)
    assert call(lr=float("nan")) == -1
    assert call(nbytes=need - 1) == -3
    assert call(ws_=ctypes.c_void_p((1 << 20) + 8)) == -1
    assert call(s=_shape(moe, T=64, routed=moe.MOE_MXFP4)) == -2
    no_dx = moe.MoeGrads(*([1 << 20] * len(moe.MoeGrads._fields_)))
    no_dx.dx = None
    assert call(g=no_dx) == -1
    no_router = moe.MoeGrads(*([1 << 20] * len(moe.MoeGrads._fields_)))
    no_router.d_w_router = None
    assert call(g=no_router) == -1


def test_training_calls_validation_on_host():
    import sparse_moe_ffn_sigmoid_amd as moe
    lib = moe.lib()
    fake = ctypes.c_void_p(1 << 20)            # never dereferenced: validation fails first
    sb = lambda **kw: lib.moe_saved_activations_bytes(ctypes.byref(_shape(moe, **kw)))
    assert sb(T=64) > 0 and sb(T=0) > 0
    assert sb(routed=moe.MOE_MXFP4) == 0 and sb(act=moe.MOE_F32, routed=moe.MOE_F32) == 0
    assert sb(T=-1) == 0 and sb(T=(1 << 20) + 1) == 0
    sh = _shape(moe, T=64)
    wts = moe.MoeWeights(*([1 << 20] * len(moe.MoeWeights._fields_)))
    need_f = lib.moe_forward_workspace_bytes(ctypes.byref(sh))
    need_s = sb(T=64)
    fwd = lambda saved=fake, nsaved=need_s, s=sh: lib.moe_latent_forward_train(
        ctypes.byref(s), ctypes.byref(wts), fake, fake, fake, None, None, fake, fake, fake, fake,
        saved, nsaved, fake, need_f, None)
    assert fwd(saved=None) == -1
    assert fwd(saved=ctypes.c_void_p((1 << 20) + 8)) == -1
    assert fwd(nsaved=need_s - 1) == -3
    assert fwd(s=_shape(moe, T=64, routed=moe.MOE_MXFP4)) == -2
    grads = moe.MoeGrads(*([1 << 20] * len(moe.MoeGrads._fields_)))
    need_b = lib.moe_backward_workspace_bytes(ctypes.byref(sh))
    bwd = lambda saved=fake, nsaved=need_s, sgd=0, lr=0.1, g=grads: lib.moe_latent_backward_train(
        ctypes.byref(sh), ctypes.byref(wts), fake, fake, fake, fake, fake, saved, nsaved,
        ctypes.byref(g), sgd, ctypes.c_float(lr), fake, need_b, None)
    assert bwd(saved=None) == -1
    assert bwd(nsaved=need_s - 1) == -3
    assert bwd(sgd=2) == -1
    assert bwd(sgd=1, lr=float("nan")) == -1
    no_gate = moe.MoeGrads(*([1 << 20] * len(moe.MoeGrads._fields_)))
    no_gate.d_w_gate = None
    assert bwd(g=no_gate) == -1                                 # plain gradients need all of them
