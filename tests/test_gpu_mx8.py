"""moe_mxfp8_quantize (the W4A8 path's on-the-fly MXFP8 rounding of the
routed experts' inputs) against the oracle's MXFP8 quantiser, bit for bit:
codes and scale bytes, on blocks built to hit every branch of the format
(OCP Microscaling v1.0: E4M3 elements, one E8M0 scale per 32 elements)."""
import numpy as np
import pytest
import torch

from layer_cases import announce
from oracle import layer as olayer

pytestmark = pytest.mark.gpu

E4M3_NORMAL = [m / 8.0 * 2.0 ** e for e in range(-6, 9) for m in range(8, 16)
               if m / 8.0 * 2.0 ** e <= 448.0]
E4M3_SUB = [m * 2.0 ** -9 for m in range(0, 8)]


def bf16_round(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def blocks(rng):
    """float64 blocks of 32 values, each exactly representable in bf16."""
    out = []
    grid = np.array(E4M3_SUB + E4M3_NORMAL)
    for X in (-20, -3, 0, 5, 40):
        scale = 2.0 ** X
        # amax exactly 256 * 2^X (a power of two), the rest at midpoints between
        # neighbouring E4M3 values: every element is a tie
        mids = (grid[1:] + grid[:-1]) / 2
        b = np.concatenate([[256.0], rng.choice(mids, 31)]) * scale
        b *= rng.choice([-1.0, 1.0], 32)
        out.append(b)
        # exactly representable values, no rounding at all
        out.append(np.concatenate([[-256.0], rng.choice(grid, 31)]) * scale)
    # saturation: amax / 2^X in (448, 512): 1.75, 1.8125, 1.9375, 1.9921875 x 2^8
    for top in (1.75, 1.8125, 1.9375, 1.9921875):
        b = rng.standard_normal(32) * 50
        b[:4] = [top * 256, -top * 256, 1.875 * 256, -1.8125 * 256]
        out.append(bf16_round(b))
    # all-zero blocks, with and without the sign bit
    out.append(np.zeros(32))
    out.append(-np.zeros(32))
    # amax a power of two, others below the E4M3 subnormal range after scaling
    b = np.full(32, 2.0 ** -30)
    b[0] = 2.0 ** 3
    b[1::2] *= -1
    out.append(b)
    # bf16 subnormal inputs (below 2^-126): the scale byte clamps to 0
    sub = np.array([m * 2.0 ** -133 for m in range(1, 128)])
    out.append(rng.choice(sub, 32) * rng.choice([-1.0, 1.0], 32))
    out.append(np.concatenate([[2.0 ** -119 * 1.5], rng.choice(sub, 31)]))   # exponent -119: byte 0
    out.append(np.concatenate([[2.0 ** -118], rng.choice(sub, 31)]))         # byte 1
    # the largest bf16 magnitudes: byte 246
    out.append(bf16_round(np.concatenate([[3.3e38, -3.0e38], rng.standard_normal(30) * 1e37])))
    # ordinary data over a wide range of magnitudes
    for e in range(-130, 128, 7):
        out.append(bf16_round(rng.standard_normal(32) * 2.0 ** e))
    return out


@pytest.mark.parametrize("K", [32, 256, 7168])
def test_mxfp8_quantize_bit_exact(K):
    import sparse_moe_ffn_sigmoid_amd as moe
    rng = np.random.default_rng(K)
    blk = blocks(rng)
    per_row = K // 32
    rows = (len(blk) + per_row - 1) // per_row + 3
    extra = rows * per_row - len(blk)
    blk += [bf16_round(rng.standard_normal(32)) for _ in range(extra)]
    rng.shuffle(blk)
    v = np.concatenate(blk).reshape(rows, K)
    x = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(x.to(torch.float64).numpy(), v)   # every value is a bf16 value
    announce(f"mxfp8 quantize rows={rows} K={K}")
    codes, scales = moe.mxfp8_quantize(x.cuda())
    torch.cuda.synchronize()
    want_c, want_s = olayer.mxfp8_quantize(x.to(torch.float64).numpy())
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    bad = np.argwhere(got_s != want_s)
    assert bad.size == 0, f"scale bytes differ at {bad[:5].tolist()}"
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, (f"codes differ at {bad[:5].tolist()}: got "
                           f"{got_c[tuple(bad[0])]:#x} want {want_c[tuple(bad[0])]:#x}")
    # the byte range the blocks reach: 0 (clamped) through 246 (largest bf16)
    assert want_s.min() == 0 and want_s.max() == 246


def test_mxfp8_quantize_empty():
    import sparse_moe_ffn_sigmoid_amd as moe
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    codes, scales = moe.mxfp8_quantize(x)
    assert codes.shape == (0, 64) and scales.shape == (0, 2)


# --- MXFP4 activations (the W4A4 path's rounding of z and h) ---------------

E2M1_GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def blocks4(rng):
    """float64 blocks of 32 bf16 values for the E2M1 quantiser."""
    out = []
    grid = np.array(E2M1_GRID)
    mids = (grid[1:] + grid[:-1]) / 2                      # .25 .75 1.25 1.75 2.5 3.5 5
    for X in (-20, -3, 0, 5, 40):
        scale = 2.0 ** X
        # amax 4 * 2^X (a power of two): every other element sits on a midpoint
        b = np.concatenate([[4.0], rng.choice(mids, 31)]) * scale
        out.append(b * rng.choice([-1.0, 1.0], 32))
        out.append(np.concatenate([[-4.0], rng.choice(grid, 31)]) * scale)
        # amax in (6, 8) * 2^X: saturation to 6, and values between 5 and 6
        b = np.concatenate([[7.5, -6.5, 5.5, -5.25, 5.0, 6.0], rng.choice(mids, 26)]) * scale
        out.append(b)
    out.append(np.zeros(32))
    out.append(-np.zeros(32))
    b = np.full(32, 2.0 ** -30)
    b[0] = 2.0 ** 3
    b[1::2] *= -1
    out.append(b)
    sub = np.array([m * 2.0 ** -133 for m in range(1, 128)])
    out.append(rng.choice(sub, 32) * rng.choice([-1.0, 1.0], 32))
    out.append(np.concatenate([[2.0 ** -125 * 1.5], rng.choice(sub, 31)]))   # exponent -125: byte 0
    out.append(np.concatenate([[2.0 ** -124], rng.choice(sub, 31)]))         # byte 1
    out.append(bf16_round(np.concatenate([[3.3e38, -3.0e38], rng.standard_normal(30) * 1e37])))
    for e in range(-130, 128, 7):
        out.append(bf16_round(rng.standard_normal(32) * 2.0 ** e))
    return out


@pytest.mark.parametrize("K", [32, 256, 7168])
def test_mxfp4_quantize_bit_exact(K):
    import sparse_moe_ffn_sigmoid_amd as moe
    rng = np.random.default_rng(100 + K)
    blk = blocks4(rng)
    per_row = K // 32
    rows = (len(blk) + per_row - 1) // per_row + 3
    blk += [bf16_round(rng.standard_normal(32)) for _ in range(rows * per_row - len(blk))]
    rng.shuffle(blk)
    v = np.concatenate(blk).reshape(rows, K)
    x = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    assert np.array_equal(x.to(torch.float64).numpy(), v)   # every value is a bf16 value
    announce(f"mxfp4 quantize rows={rows} K={K}")
    codes, scales = moe.mxfp4_quantize(x.cuda())
    torch.cuda.synchronize()
    want_c, want_s = olayer.mxfp4_act_quantize(x.to(torch.float64).numpy())
    packed, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    got_c = np.empty((rows, K), np.uint8)
    got_c[:, 0::2] = packed & 0xF
    got_c[:, 1::2] = packed >> 4
    bad = np.argwhere(got_s != want_s)
    assert bad.size == 0, f"scale bytes differ at {bad[:5].tolist()}"
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, (f"codes differ at {bad[:5].tolist()}: got "
                           f"{got_c[tuple(bad[0])]:#x} want {want_c[tuple(bad[0])]:#x}")
    assert want_s.min() == 0 and want_s.max() == 252
