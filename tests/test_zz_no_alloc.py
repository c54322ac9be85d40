"""moe_forward_noalloc (for callers that cannot allocate device memory)
through the C ABI against moe_forward with its own workspace: the same
kernels on the library's fixed scratch, so the outputs must be identical bit
for bit (and within the oracle's bar); two calls in a row, the second with
fewer tokens, so the scratch is reused with another layout."""

import ctypes

import numpy as np
import pytest
import torch

import expert_gemms_amd as moe
from expert_gemms_amd import _lib
from oracle.moe import moe_reference
from synth import MoEConfig, gen_routing, gen_x_bf16, gen_w2_input_scale, bf16_bits
from tests.gpu_util import dev, run_layer, x_dev
from tests.helpers import check_layer, make_weights

pytestmark = pytest.mark.gpu

CFGS = {
    "mxfp4": MoEConfig("noalloc_mxfp4", 90, "mxfp4", 40, 512, 256, 32, 4, routing="softmax_uniform"),
    "bf16": MoEConfig("noalloc_bf16", 91, "bf16", 60, 512, 384, 8, 2, routing="softmax_uniform"),
    "nvfp4": MoEConfig("noalloc_nvfp4", 92, "nvfp4", 50, 512, 256, 16, 6, routing="zipf"),
}


def noalloc(layer, T, x, ids, wts, out):
    """One moe_forward_noalloc call through ctypes; returns its status."""
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    lib = moe.lib_handle()
    st = lib.moe_forward_noalloc(_lib.FMT[layer.fmt], T, layer.hidden, layer.inter, layer.top_k, 0,
                                 layer.num_local_experts, layer.num_shared, 0, None, None, p(x), p(ids), p(wts),
                                 p(layer.w13_k), p(layer.w13_sf_k), p(layer.w2_k), p(layer.w2_sf_k), p(layer.w13_gs),
                                 p(layer.w2_gs), ctypes.c_float(layer.l2_activation_scale), p(out),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


@pytest.mark.parametrize("fmt", sorted(CFGS))
def test_noalloc_equals_moe_forward_twice(fmt):
    cfg = CFGS[fmt]
    x = bf16_bits(gen_x_bf16(cfg))
    ids, wts = gen_routing(cfg)
    w = make_weights(cfg)
    w2in = gen_w2_input_scale(cfg) if fmt == "nvfp4" else None
    g2 = 1.0 if w2in is None else float(w2in.max())
    _, layer = run_layer(fmt, x, ids, wts, w, w2_input_scale=w2in)
    # second call: fewer tokens, taken from the end (other routing)
    for T, sl in ((cfg.T, slice(0, cfg.T)), (7, slice(cfg.T - 7, cfg.T))):
        xd, idd, wd = x_dev(x[sl]), dev(ids[sl].astype(np.int32)), dev(wts[sl].astype(np.float32))
        out = torch.full((T, cfg.H), float("nan"), dtype=torch.bfloat16, device="cuda")
        assert noalloc(layer, T, xd, idd, wd, out) == _lib.OK
        ref_out = layer.forward(xd, idd, wd)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), (fmt, T)
        y = out.float().cpu().numpy().astype(np.float64)
        ref = moe_reference(fmt, x[sl], ids[sl], wts[sl], w, l2_activation_scale=g2)
        rel, excess, _ = check_layer(fmt, y, ref, x[sl], ids[sl], wts[sl], w, g2=g2)
        assert excess <= 0, (fmt, T, rel)


def test_noalloc_rejects_a_layer_too_large_for_its_scratch():
    cfg = CFGS["bf16"]
    x = bf16_bits(gen_x_bf16(cfg))
    ids, wts = gen_routing(cfg)
    _, layer = run_layer("bf16", x, ids, wts, make_weights(cfg))
    T = 20000                                        # > 64 MiB of intermediate rows
    big_x = torch.zeros((T, cfg.H), dtype=torch.bfloat16, device="cuda")
    big_ids = torch.zeros((T, cfg.top_k), dtype=torch.int32, device="cuda")
    big_w = torch.zeros((T, cfg.top_k), dtype=torch.float32, device="cuda")
    out = torch.zeros((T, cfg.H), dtype=torch.bfloat16, device="cuda")
    assert noalloc(layer, T, big_x, big_ids, big_w, out) == _lib.E_TOO_LARGE
    torch.cuda.synchronize()
    assert not out.any()                             # nothing ran
