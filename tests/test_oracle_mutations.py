"""The pins have teeth: plant a plausible mistake in the oracle (on the CPU,
via monkeypatch) and check that one of the independent pins rejects it."""

import numpy as np
import pytest

from oracle import codecs, quant
from oracle import moe as M
from synth import gen_x_bf16, gen_routing, bf16_bits
from tests.helpers import make_weights
from tests.test_oracle_moe import dense_top1, small_cfg


def _dense_pin_holds(fmt):
    cfg = small_cfg(fmt, k=1)
    x = bf16_bits(gen_x_bf16(cfg))
    ids, _ = gen_routing(cfg)
    w = make_weights(cfg)
    y = M.moe_reference(fmt, x, ids, np.ones(ids.shape, np.float32), w, l2_activation_scale=0.013)
    ref = dense_top1(fmt, x, ids, w, 0.013)
    return np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


MUTATIONS = {
    "gate_up_swapped": ("activation", lambda orig: (lambda g, u, *a, **k: orig(u, g, *a, **k))),
    "sigmoid_sign": ("sigmoid", lambda orig: (lambda z: orig(-z))),
    "l2_quant_dropped": ("quantize_l2_input", lambda orig: (lambda fmt, a, s=1.0: np.asarray(a, np.float64))),
    "wrong_expert": ("dequant_weight", lambda orig: (lambda fmt, w, n, e: orig(fmt, w, n, (e + 1) % w[n].shape[0]))),
    "w13_transposed_halves": ("dequant_weight", lambda orig: (
        lambda fmt, w, n, e: np.roll(orig(fmt, w, n, e), orig(fmt, w, n, e).shape[0] // 2, 0)
        if n == "w13" else orig(fmt, w, n, e))),
    "x_quant_dropped": ("quantize_x", lambda orig: (
        lambda fmt, xb: codecs.bf16_decode(xb))),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
@pytest.mark.parametrize("fmt", ["bf16", "mxfp8", "nvfp4"])
def test_dense_pin_rejects_mutation(monkeypatch, name, fmt):
    attr, make = MUTATIONS[name]
    if name == "x_quant_dropped" and fmt == "bf16":
        pytest.skip("BF16 dispatch has no quantisation to drop")
    monkeypatch.setattr(M, attr, make(getattr(M, attr)))
    assert not _dense_pin_holds(fmt)


def test_quant_pins_reject_floor_scale(monkeypatch):
    """OCP's floor-style exponent (which clips) instead of the no-clip scale
    fails the minimality pin."""
    def floor_codes(amax, elem):
        amax = np.asarray(amax, np.float64)
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - (8 if elem == "e4m3" else 2)
        return np.where(amax > 0, np.clip(127 + e, 1, 254), 0).astype(np.uint8)
    monkeypatch.setattr(quant, "mx_scale_codes", floor_codes)
    v = np.full((1, 32), 500.0, np.float32)                   # amax 500 > 448 * 2^0
    _, c = quant.mx_quantize(v, "e4m3")
    assert not 500.0 <= 448.0 * 2.0 ** (int(c[0, 0]) - 127)
