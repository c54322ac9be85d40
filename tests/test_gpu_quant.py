"""The HIP quantisers against the oracle's, bit-exact: dispatch quantisation
of BF16 x (the kernel moe_forward runs for a1) and the weight casts."""

import numpy as np
import pytest
import torch

import expert_gemms_amd as moe
from oracle import codecs, quant
from tests.gpu_util import dev, x_dev

pytestmark = pytest.mark.gpu


def special_x(T, H, seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, H)) * np.exp2(rng.integers(-20, 20, (T, 1)))).astype(np.float32)
    x[0] = 0.0                                       # an all-zero row
    x[1, :32] = 0.0                                  # an all-zero block
    x[2, :32] = 0.0
    x[2, 5] = 1e-40                                  # a block with a subnormal amax
    x[3, :64] = np.float32(448.0)                    # exact fmax
    x[4, 7] = -np.float32(1.75 * 2 ** 5)             # m = 1.75 boundary
    x[5, 9] = np.float32(1.5 * 2 ** -3)              # m = 1.5 boundary
    x[6, 3] = -0.0
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return bits


@pytest.mark.parametrize("T,H", [(7, 256), (130, 1024), (64, 7168)])
def test_quantize_x_mxfp8_bit_exact(T, H):
    xb = special_x(T, H, T + H)
    codes = torch.empty((T, H), dtype=torch.uint8, device="cuda")
    sf = torch.empty((T, H // 32), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_x("mxfp8", T, H, x_dev(xb), codes, sf)
    torch.cuda.synchronize()
    q, c = quant.mx_quantize(codecs.bf16_decode(xb).astype(np.float32), "e4m3")
    assert np.array_equal(sf.cpu().numpy(), c)
    assert np.array_equal(codes.cpu().numpy(), q)


@pytest.mark.parametrize("T,H", [(7, 256), (130, 2048), (9, 2304), (7, 6144)])
def test_quantize_x_nvfp4_bit_exact(T, H):
    xb = special_x(T, H, 3 * T + H)
    codes = torch.empty((T, H // 2), dtype=torch.uint8, device="cuda")
    sf = torch.empty((T, H // 16), dtype=torch.uint8, device="cuda")
    ts = torch.empty((T,), dtype=torch.float32, device="cuda")
    moe.moe_quantize_x("nvfp4", T, H, x_dev(xb), codes, sf, ts)
    torch.cuda.synchronize()
    x32 = codecs.bf16_decode(xb).astype(np.float32)
    g = quant.nvfp4_global_scale(np.abs(x32).max(axis=1))
    q, bs = quant.nvfp4_quantize(x32, g)
    assert np.array_equal(ts.cpu().numpy(), g)
    assert np.array_equal(sf.cpu().numpy(), bs)
    assert np.array_equal(codes.cpu().numpy(), codecs.fp4_pack(q))


def _bf16_bits(x32):
    return torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


def test_quantize_x_mxfp8_rounding_ties_bit_exact():
    """Every element an exact midpoint between two E4M3 codes after scaling
    (each block holds 448, so its scale is 2^0): the encoder must round each
    tie to the even code, as the oracle does."""
    mags = []
    for c in range(0x7E):                       # midpoints between codes c and c + 1
        lo, hi = (codecs.e4m3_decode(np.array([c, c + 1], dtype=np.uint8))).astype(np.float64)
        mags.append((lo + hi) / 2)
    vals = np.array(mags + [-m for m in mags], dtype=np.float64)   # 252 ties
    T, H = 2, 288
    x = np.zeros((T, H), dtype=np.float32)
    flat = np.concatenate([vals, vals[::-1]])
    pos = 0
    for t in range(T):
        for b in range(H // 32):
            x[t, 32 * b] = 448.0 if (t + b) % 2 == 0 else -448.0
            n = min(31, flat.size - pos)
            x[t, 32 * b + 1:32 * b + 1 + n] = flat[pos:pos + n]
            pos += n
    assert pos == flat.size
    xb = _bf16_bits(x)
    assert np.array_equal(codecs.bf16_decode(xb).astype(np.float32), x)    # the ties are exact in BF16
    codes = torch.empty((T, H), dtype=torch.uint8, device="cuda")
    sf = torch.empty((T, H // 32), dtype=torch.uint8, device="cuda")
    moe.moe_quantize_x("mxfp8", T, H, x_dev(xb), codes, sf)
    torch.cuda.synchronize()
    q, c = quant.mx_quantize(x, "e4m3")
    assert np.all(c == 127)
    assert np.array_equal(sf.cpu().numpy(), c)
    assert np.array_equal(codes.cpu().numpy(), q)


def test_quantize_x_nvfp4_rounding_ties_bit_exact():
    """Rows whose token scale is exactly 1 (amax 2688) and whose 16-blocks hold
    6 (block scale exactly 1) and the E2M1 midpoints of both signs: every
    element is a tie the encoder must round to the even code."""
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    T, H = 3, 256
    x = np.zeros((T, H), dtype=np.float32)
    for t in range(T):
        for b in range(H // 16 - 1):
            blk = np.concatenate([[6.0 if b % 2 else -6.0], ties, -ties, [ties[(t + b) % 7]]])
            x[t, 16 * b:16 * b + 16] = np.roll(blk, t + b)
        x[t, H - 16] = 2688.0 if t % 2 == 0 else -2688.0
    xb = _bf16_bits(x)
    assert np.array_equal(codecs.bf16_decode(xb).astype(np.float32), x)
    codes = torch.empty((T, H // 2), dtype=torch.uint8, device="cuda")
    sf = torch.empty((T, H // 16), dtype=torch.uint8, device="cuda")
    ts = torch.empty((T,), dtype=torch.float32, device="cuda")
    moe.moe_quantize_x("nvfp4", T, H, x_dev(xb), codes, sf, ts)
    torch.cuda.synchronize()
    g = quant.nvfp4_global_scale(np.abs(x).max(axis=1))
    q, bs = quant.nvfp4_quantize(x, g)
    assert np.all(g == 1.0) and np.all(bs[:, :-1] == 0x38)
    assert np.array_equal(ts.cpu().numpy(), g)
    assert np.array_equal(sf.cpu().numpy(), bs)
    assert np.array_equal(codes.cpu().numpy(), codecs.fp4_pack(q))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "nvfp4"])
def test_quantize_weights_bit_exact(fmt):
    E, R, K = 3, 96, 256
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((E, R, K)) * 0.02).astype(np.float32)
    w[1, 3, :32] = 0
    w[2] = 0                                          # an all-zero expert
    vpe = 2 if fmt != "mxfp8" else 1
    grp = 16 if fmt == "nvfp4" else 32
    codes = torch.empty((E, R, K // vpe), dtype=torch.uint8, device="cuda")
    sf = torch.empty((E, R, K // grp), dtype=torch.uint8, device="cuda")
    gs = torch.empty((E,), dtype=torch.float32, device="cuda") if fmt == "nvfp4" else None
    moe.moe_quantize_weights(fmt, E, R, K, dev(w), codes, sf, gs)
    torch.cuda.synchronize()
    if fmt == "nvfp4":
        g = quant.nvfp4_global_scale(np.abs(w).reshape(E, -1).max(axis=1))
        assert np.array_equal(gs.cpu().numpy(), g)
        q, bs = quant.nvfp4_quantize(w, np.broadcast_to(g[:, None], (E, R)))
        assert np.array_equal(sf.cpu().numpy(), bs)
        assert np.array_equal(codes.cpu().numpy(), codecs.fp4_pack(q))
    else:
        q, c = quant.mx_quantize(w, "e4m3" if fmt == "mxfp8" else "e2m1")
        assert np.array_equal(sf.cpu().numpy(), c)
        want = q if fmt == "mxfp8" else codecs.fp4_pack(q)
        assert np.array_equal(codes.cpu().numpy(), want)
