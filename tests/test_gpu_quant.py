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


@pytest.mark.parametrize("T,H", [(7, 256), (130, 2048)])
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
