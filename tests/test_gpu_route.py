"""moe_route (router top-k) against the oracle on seeded logits.

Ids are compared exactly.  Where float32 (GPU) and float64 (oracle) scores
order two candidates differently, both orders are correct: a token whose ids
differ is accepted only if every chosen expert's oracle choice score lies
within 1e-5 (relative) of the score the oracle chose at that rank, and such
tokens must be rare.  Weights: relative 2e-5 against the oracle's weights of
the ids the GPU chose.
"""

import zlib

import numpy as np
import pytest
import torch

import expert_gemms_amd as moe
from oracle.routing import route_reference, scores_of

pytestmark = pytest.mark.gpu

CASES = {
    # name: (T, E, k, scoring, bias, groups, topk_groups, renormalize, scaling, coarse logits, padding)
    "mixtral_softmax": (4096, 8, 2, "softmax", False, 1, 1, True, 1.0, False, False),
    "qwen_softmax_no_renorm": (2048, 128, 8, "softmax", False, 1, 1, False, 1.0, False, False),
    "dsv3_grouped_sigmoid_bias": (8192, 256, 8, "sigmoid", True, 8, 4, True, 2.5, False, False),
    "softmax_bias_scaled": (1000, 64, 6, "softmax", True, 1, 1, True, 1.5, False, True),
    "ties": (3000, 96, 6, "softmax", False, 1, 1, True, 1.0, True, False),
    "ties_grouped": (3000, 96, 6, "sigmoid", True, 12, 3, False, 1.0, True, True),
    "wide_1024": (512, 1024, 16, "softmax", False, 1, 1, True, 1.0, False, False),
    "odd_E_160": (777, 160, 5, "sigmoid", False, 5, 2, True, 1.0, False, False),
    "single_token": (1, 256, 8, "sigmoid", True, 8, 4, True, 2.5, False, False),
}


def _inputs(name):
    T, E, k, scoring, use_bias, G, TG, renorm, scaling, coarse, pad = CASES[name]
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if coarse:
        logits = (np.round(logits * 4) / 4).astype(np.float32)      # many exact ties
    bias = (rng.standard_normal(E) * 0.05).astype(np.float32) if use_bias else None
    if coarse and bias is not None:
        bias = (np.round(bias * 64) / 64).astype(np.float32)
    is_pad = (rng.random(T) < 0.05).astype(np.uint8) if pad else None
    return logits, bias, is_pad


@pytest.mark.parametrize("name", sorted(CASES))
def test_route_matches_oracle(name):
    T, E, k, scoring, use_bias, G, TG, renorm, scaling, coarse, pad = CASES[name]
    logits, bias, is_pad = _inputs(name)
    ids_d = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w_d = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_route(T, E, k, torch.from_numpy(logits).cuda(), ids_d, w_d,
                  bias=None if bias is None else torch.from_numpy(bias).cuda(), scoring=scoring,
                  num_groups=G, topk_groups=TG, renormalize=renorm, routed_scaling_factor=scaling,
                  is_padding=None if is_pad is None else torch.from_numpy(is_pad).cuda())
    torch.cuda.synchronize()
    ids, w = ids_d.cpu().numpy(), w_d.cpu().numpy().astype(np.float64)
    rids, rw, masked = route_reference(logits.astype(np.float64), k, scoring=scoring,
                                       bias=None if bias is None else bias.astype(np.float64),
                                       num_groups=G, topk_groups=TG, renormalize=renorm, scaling=scaling,
                                       is_padding=is_pad)
    differ = np.nonzero((ids != rids).any(axis=1))[0]
    s = scores_of(logits.astype(np.float64), scoring)
    choice = s + (0.0 if bias is None else bias.astype(np.float64)[None, :])
    for t in differ:
        assert len(set(ids[t].tolist())) == k and (ids[t] >= 0).all(), (t, ids[t])
        got, want = choice[t, ids[t]], np.take(masked[t], rids[t])
        assert np.all(np.abs(got - want) <= 1e-5 * np.maximum(1.0, np.abs(want))), (t, ids[t], rids[t], got, want)
    assert len(differ) <= max(2, T // 1000), f"{len(differ)} tokens ordered differently"
    # weights of the ids the GPU chose
    sel = np.take_along_axis(s, np.maximum(ids, 0).astype(np.int64), axis=1)
    if renorm:
        sel = sel / sel.sum(axis=1, keepdims=True)
    ew = sel * scaling
    if is_pad is not None:
        p = is_pad.astype(bool)
        assert (ids[p] == -1).all() and (w[p] == 0).all()
        ew[p] = 0.0
    assert np.allclose(w, ew, rtol=2e-5, atol=1e-7)
    print(f"{name}: {len(differ)} of {T} tokens take another valid order")


def test_route_feeds_the_layer():
    """Padding tokens routed by moe_route come out of moe_forward as zeros."""
    from tests.gpu_util import run_layer
    from tests.helpers import make_weights
    from synth import MoEConfig, gen_x_bf16, bf16_bits
    cfg = MoEConfig("route_layer", 30, "bf16", 64, 256, 256, 8, 2)
    x = bf16_bits(gen_x_bf16(cfg))
    logits = np.random.default_rng(3).standard_normal((64, 8)).astype(np.float32)
    is_pad = np.zeros(64, dtype=np.uint8)
    is_pad[[5, 40]] = 1
    ids_d = torch.empty((64, 2), dtype=torch.int32, device="cuda")
    w_d = torch.empty((64, 2), dtype=torch.float32, device="cuda")
    moe.moe_route(64, 8, 2, torch.from_numpy(logits).cuda(), ids_d, w_d,
                  is_padding=torch.from_numpy(is_pad).cuda())
    y, _ = run_layer("bf16", x, ids_d.cpu().numpy(), w_d.cpu().numpy(), make_weights(cfg))
    assert not y[[5, 40]].any() and y[[0, 6, 41]].any()
