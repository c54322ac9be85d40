"""Pins of the oracle's output-side variants: the post-expert RMSNorm and
the routing weight applied on the input."""

import numpy as np
import pytest
import torch

from oracle import moe as M
from synth import gen_routing, gen_x_bf16, bf16_bits
from tests.helpers import make_weights
from tests.test_oracle_moe import dense_top1, small_cfg

FMTS = ["bf16", "mxfp8", "mxfp4", "nvfp4"]


def test_rms_norm_against_torch_and_closed_forms():
    rng = np.random.default_rng(4)
    y = rng.standard_normal((9, 96))
    gamma = rng.uniform(0.5, 1.5, 96)
    got = M.post_expert_norm(y, gamma, 1e-6)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(y), (96,), torch.from_numpy(gamma), 1e-6).numpy()
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)
    # a constant row c: c / sqrt(c^2 + eps) * gamma
    c = np.full((1, 8), -3.0)
    assert np.allclose(M.post_expert_norm(c, np.ones(8), 0.5), -3.0 / np.sqrt(9.5))
    # scale invariance without eps
    assert np.allclose(M.post_expert_norm(7.5 * y, gamma, 0.0), M.post_expert_norm(y, gamma, 0.0), rtol=1e-12)


@pytest.mark.parametrize("fmt", FMTS)
def test_norm_applies_to_the_layer_output(fmt):
    cfg = small_cfg(fmt, k=2, n_sh=1)
    x = bf16_bits(gen_x_bf16(cfg))
    ids, wts = gen_routing(cfg)
    w = make_weights(cfg)
    gamma = np.linspace(0.5, 2.0, cfg.H)
    y = M.moe_reference(fmt, x, ids, wts, w, num_shared=1, l2_activation_scale=0.013)
    yn = M.moe_reference(fmt, x, ids, wts, w, num_shared=1, l2_activation_scale=0.013, norm=(gamma, 1e-5))
    ms = np.mean(y * y, axis=1, keepdims=True)
    assert np.allclose(yn, y / np.sqrt(ms + 1e-5) * gamma, rtol=1e-12)


@pytest.mark.parametrize("fmt", FMTS)
def test_weight_on_input_is_a_dense_mlp_of_the_scaled_input(fmt):
    cfg = small_cfg(fmt, k=1)
    x = bf16_bits(gen_x_bf16(cfg))
    ids, _ = gen_routing(cfg)
    wts = np.random.default_rng(2).uniform(0.2, 1.0, ids.shape).astype(np.float32)
    w = make_weights(cfg)
    y = M.moe_reference(fmt, x, ids, wts, w, l2_activation_scale=0.013, router_weight_on_input=True)
    # scaled input built by another route: torch bfloat16 multiply-and-round
    xs = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float()
          * torch.from_numpy(wts)).bfloat16().view(torch.int16).numpy().view(np.uint16)
    ref = dense_top1(fmt, xs, ids, w, 0.013)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # weight 1 is the plain layer
    ones = np.ones_like(wts)
    assert np.array_equal(M.moe_reference(fmt, x, ids, ones, w, l2_activation_scale=0.013, router_weight_on_input=True),
                          M.moe_reference(fmt, x, ids, ones, w, l2_activation_scale=0.013))


def test_weight_on_input_needs_top1_without_shared():
    cfg = small_cfg("bf16", k=2)
    x = bf16_bits(gen_x_bf16(cfg))
    ids, wts = gen_routing(cfg)
    with pytest.raises(ValueError):
        M.moe_reference("bf16", x, ids, wts, make_weights(cfg), router_weight_on_input=True)
