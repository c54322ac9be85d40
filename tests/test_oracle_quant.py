"""Pins of the oracle's block quantisers: scale minimality found by exhaustive
exponent search, round-trip idempotence, half-ulp error bounds, zero blocks,
torch's float8 rounding for the NVFP4 block scale, and the special case where
NVFP4 and MXFP4 must agree code for code."""

import numpy as np
import pytest
import torch

from oracle import codecs, quant


def _blocks(rng, n, group, spread=20):
    mag = np.exp2(rng.uniform(-spread, spread, (n, 1)))
    v = (rng.standard_normal((n, group)) * mag).astype(np.float32)
    # exact boundary amaxes: m * 2^p with m at the E4M3 / E2M1 thresholds
    for i, m in enumerate((1.0, 1.5, 1.75, 1.7500001, 1.5000001, 1.9999999)):
        v[i] = 0
        v[i, i % group] = np.float32(m * 2.0 ** (i - 3))
    return v


@pytest.mark.parametrize("elem,fmax", [("e4m3", 448.0), ("e2m1", 6.0)])
def test_mx_scale_is_smallest_nonclipping_power_of_two(elem, fmax):
    rng = np.random.default_rng(10)
    v = _blocks(rng, 3000, 32)
    _, c = quant.mx_quantize(v, elem)
    amax = np.abs(v.astype(np.float64)).max(axis=1)
    for a, code in zip(amax, c[:, 0]):
        # brute force: walk e up from far below until amax <= fmax * 2**e
        e = -200
        while not a <= fmax * 2.0 ** e:
            e += 1
        assert code == min(max(127 + e, 1), 254)


@pytest.mark.parametrize("elem", ["e4m3", "e2m1"])
def test_mx_roundtrip_idempotent_and_half_ulp(elem):
    rng = np.random.default_rng(11)
    v = _blocks(rng, 2000, 32, spread=10).reshape(-1, 64)
    q, c = quant.mx_quantize(v, elem)
    d = quant.mx_dequantize(q, c, elem)
    # values are idempotent; codes need not be, since a block amax that rounds
    # up onto fmax * 2^e re-quantises with the next smaller scale
    q2, c2 = quant.mx_quantize(d.astype(np.float32), elem)
    assert np.array_equal(quant.mx_dequantize(q2, c2, elem), d)
    # error <= half a unit in the last place of the element's own binade
    s = np.repeat(codecs.ue8m0_decode(c), 32, axis=1)
    x = np.abs(v.astype(np.float64)) / s
    mbits, emin = (3, -6) if elem == "e4m3" else (1, 0)
    e = np.maximum(np.floor(np.log2(np.where(x > 0, x, 1.0))), emin)
    ulp = np.exp2(e - mbits)
    assert np.all(np.abs(v - d) <= 0.5 * ulp * s * (1 + 1e-12))


def test_mx_zero_block_and_small_magnitudes():
    v = np.zeros((2, 64), dtype=np.float32)
    v[1, 40] = np.float32(1e-40)              # subnormal float32 input
    q, c = quant.mx_quantize(v, "e4m3")
    assert c[0].tolist() == [0, 0] and not q[0].any()
    assert c[1, 0] == 0 and c[1, 1] == 1       # clamped to the smallest code
    assert quant.mx_dequantize(q, c, "e4m3")[0].sum() == 0


def test_nvfp4_block_scale_matches_torch_float8():
    """bs = E4M3(amax16 / (6 g)) with float32 arithmetic: recompute it with
    torch float32 tensors and torch's own float8 cast."""
    rng = np.random.default_rng(12)
    v = _blocks(rng, 4000, 16, spread=6).reshape(-1, 64)
    g = (np.abs(v).max(axis=1) / np.float32(2688.0)).astype(np.float32)
    _, bs = quant.nvfp4_quantize(v, g)
    vt = torch.from_numpy(v).view(-1, 4, 16)
    amax = vt.abs().amax(-1)
    gt = torch.from_numpy(g)[:, None]
    t = amax / (6.0 * gt)
    ref = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(bs, ref)


def test_nvfp4_elements_are_nearest_e2m1_of_float32_product():
    rng = np.random.default_rng(13)
    v = _blocks(rng, 1000, 16, spread=6).reshape(-1, 32)
    g = np.full(v.shape[0], np.float32(0.01))
    q, bs = quant.nvfp4_quantize(v, g)
    bsv = torch.from_numpy(bs).view(torch.float8_e4m3fn).float()        # [n, 2]
    denom = bsv * torch.from_numpy(g)[:, None]
    r = 1.0 / denom
    prod = (torch.from_numpy(v).view(-1, 2, 16) * r[..., None]).numpy()
    mags = codecs.e2m1_decode(np.arange(8, dtype=np.uint8))
    got = codecs.e2m1_decode(q).reshape(prod.shape)
    a = np.minimum(np.abs(prod.astype(np.float64)), 6.0)
    d = np.abs(mags[None, None, None, :] - a[..., None])
    nearest = mags[d.argmin(-1)]
    # ties (exact midpoints) resolve to the even code; rare with random data
    tie = np.sort(d, -1)[..., 1] == d.min(-1)
    ok = (np.abs(got) == nearest) | tie
    ok &= (np.signbit(got) == np.signbit(prod)) | (got == 0)
    zero_blk = (bsv == 0).numpy()[..., None]
    assert np.all(ok | zero_blk)


def test_nvfp4_equals_mxfp4_when_scales_are_powers_of_two():
    """Two 16-blocks each with amax exactly 6 * 2^p: MXFP4 picks scale 2^p for
    the 32-block, NVFP4 with a power-of-two global g picks bs * g = 2^p for both
    16-blocks, so the element codes must agree code for code."""
    rng = np.random.default_rng(14)
    n = 500
    p = rng.integers(-6, 6, n)
    v = rng.uniform(-1, 1, (n, 32)) * 6.0
    v[:, 3] = 6.0
    v[:, 20] = -6.0
    v = (v * np.exp2(p)[:, None]).astype(np.float32)
    for gexp in (-2, 0, 2):          # keeps bs = 2^(p - gexp) inside E4M3
        g = np.full(n, np.float32(2.0 ** gexp))
        qn, bs = quant.nvfp4_quantize(v, g)
        qm, c = quant.mx_quantize(v, "e2m1")
        assert np.array_equal(c[:, 0], 127 + p)
        assert np.array_equal(codecs.e4m3_decode(bs), np.exp2(p - gexp)[:, None].repeat(2, 1))
        assert np.array_equal(qn, qm)


def test_nvfp4_roundtrip_error_bound_and_zero():
    rng = np.random.default_rng(15)
    v = rng.standard_normal((300, 64)).astype(np.float32)
    v[0] = 0
    g = quant.nvfp4_global_scale(np.abs(v).max(axis=1))
    assert g[0] == 1.0
    assert np.array_equal(g[1:], (np.abs(v[1:]).max(axis=1) / np.float32(2688.0)).astype(np.float32))
    q, bs = quant.nvfp4_quantize(v, g)
    d = quant.nvfp4_dequantize(q, bs, g)
    assert not d[0].any()
    scale = np.repeat(codecs.e4m3_decode(bs), 16, axis=1) * g[:, None]
    # grid spacing of E2M1 is at most 2 (between 4 and 6); saturation at 6
    # costs at most 6 * 2^-4 (the E4M3 half-ulp) -> |err| <= 1 * scale
    assert np.all(np.abs(v - d) <= scale * (1 + 1e-9))
