"""The boundary-decision rule of tests/helpers.check_layer (CPU): a token
whose L2 input took the other valid quantisation of a boundary value is
accepted; other differences are not."""

import numpy as np
import pytest

from oracle.moe import moe_reference, quantize_x, dequant_weight
from synth import MoEConfig, gen_routing, gen_x_bf16, bf16_bits
from tests import helpers
from tests.helpers import check_layer, make_weights

CFG = {fmt: MoEConfig(f"rule_{fmt}", 40 + i, fmt, 12, 256, 64, 4, 2, routing="softmax_uniform")
       for i, fmt in enumerate(["mxfp8", "mxfp4", "nvfp4"])}


# how much the evaluation-error bound is widened so that this small case has
# a few boundary decisions per token (the MX formats' bound, which carries
# the scaled MFMA's per-step term, is wide already)
WIDEN = {"mxfp8": 0.25, "mxfp4": 0.5, "nvfp4": 2.0 ** 4}
WIDEN_MANY = {"mxfp8": 2.0, "mxfp4": 4.0, "nvfp4": 2.0 ** 9}


def _setup(fmt, monkeypatch, widen=None):
    widen = WIDEN[fmt] if widen is None else widen
    cfg = CFG[fmt]
    x = bf16_bits(gen_x_bf16(cfg))
    ids, wts = gen_routing(cfg)
    w = make_weights(cfg)
    g2 = 0.02 if fmt == "nvfp4" else 1.0
    ref = moe_reference(fmt, x, ids, wts, w, l2_activation_scale=g2)
    # scale the evaluation-error bound so that some decisions count as
    # boundary decisions in this small case
    real = helpers._act_error
    monkeypatch.setattr(helpers, "_act_error",
                        lambda W13, xs, act, fmt="mxfp8": (lambda a, da: (a, da * widen))(*real(W13, xs, act, fmt)))
    return cfg, x, ids, wts, w, g2, ref


def _largest_decision(fmt, x, ids, wts, w, g2):
    """(token, change of the output) of the boundary decision that moves the
    output most, among tokens with between 1 and 14 such decisions."""
    best = None
    for t in range(ids.shape[0]):
        xs = quantize_x(fmt, x[t:t + 1])[0]
        found = []
        for j, e in enumerate(ids[t]):
            W13, W2 = dequant_weight(fmt, w, "w13", e), dequant_weight(fmt, w, "w2", e)
            a, da = helpers._act_error(W13, xs, {}, fmt)
            for off, dv in helpers.decision_alternatives(fmt, a, da, g2):
                found.append(wts[t, j] * (W2[:, off:off + dv.size] @ dv))
        if 1 <= len(found) <= 14:
            for dy in found:
                if best is None or np.abs(dy).max() > np.abs(best[1]).max():
                    best = (t, dy)
    if best is None:
        pytest.skip("no boundary decision in this case")
    return best


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "nvfp4"])
def test_other_valid_decision_is_accepted(fmt, monkeypatch):
    cfg, x, ids, wts, w, g2, ref = _setup(fmt, monkeypatch)
    t, dy = _largest_decision(fmt, x, ids, wts, w, g2)
    y = ref.copy()
    y[t] += dy
    rel, excess, rescued = check_layer(fmt, y, ref, x, ids, wts, w, g2=g2)
    assert excess <= 0, (rel, excess)
    # if the flip alone crosses the plain bar, the rule is what accepts it
    assert rescued == (1 if helpers.check_output(fmt, y, ref)[1] > 0 else 0)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4", "nvfp4"])
def test_other_differences_are_rejected(fmt, monkeypatch):
    cfg, x, ids, wts, w, g2, ref = _setup(fmt, monkeypatch)
    rms = np.sqrt(np.mean(ref ** 2))
    for bad in (lambda y: y.__setitem__((3, 17), y[3, 17] + 0.1 * rms),     # one wrong element
                lambda y: y.__setitem__(5, y[5] * 1.2)):                    # one token scaled
        y = ref.copy()
        bad(y)
        assert check_layer(fmt, y, ref, x, ids, wts, w, g2=g2)[1] > 0


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_greedy_search_accepts_valid_flips(fmt, monkeypatch):
    """Tokens with more boundary decisions than can be enumerated: two valid
    flips applied together are still found."""
    cfg, x, ids, wts, w, g2, ref = _setup(fmt, monkeypatch, widen=WIDEN_MANY[fmt])
    for t in range(ids.shape[0]):
        xs = quantize_x(fmt, x[t:t + 1])[0]
        found = []
        for j, e in enumerate(ids[t]):
            W13, W2 = dequant_weight(fmt, w, "w13", e), dequant_weight(fmt, w, "w2", e)
            a, da = helpers._act_error(W13, xs, {}, fmt)
            for off, dv in helpers.decision_alternatives(fmt, a, da, g2):
                found.append(wts[t, j] * (W2[:, off:off + dv.size] @ dv))
        if len(found) > 12:
            break
    else:
        pytest.skip("no token with many boundary decisions")
    big = sorted(found, key=lambda d: -np.abs(d).max())[:2]
    y = ref.copy()
    y[t] += big[0] + big[1]
    assert check_layer(fmt, y, ref, x, ids, wts, w, g2=g2)[1] <= 0
