"""moe_forward (the whole HIP path: a1-a7) against the oracle, element by
element, on seeded inputs that span several tiles and ragged tails.

Bar (tests/helpers.check_output): |y_gpu - y_oracle| <= tol * RMS(y_oracle)
+ half a BF16 ulp of y_oracle, tol = 1e-2 for BF16 and 3e-2 for MX/NVFP4; a
token over it is accepted only if the oracle, recomputed with the other valid
choice of its L2-input quantisation decisions that lie on a boundary, meets it
(tests/helpers.check_layer).
"""

import numpy as np
import pytest
import torch

from oracle.moe import moe_reference
from synth import CONFIGS, MoEConfig, gen_routing, gen_x_bf16, gen_w2_input_scale, bf16_bits
from tests.gpu_util import dev, run_layer, x_dev
from tests.helpers import check_layer, check_output, make_weights, rescue_cap

pytestmark = pytest.mark.gpu

SMALL = {
    "tiny_bf16": CONFIGS["tiny_bf16"],
    "bf16_small": MoEConfig("bf16_small", 11, "bf16", 200, 512, 384, 8, 2, routing="softmax_uniform"),
    "mxfp8_small": MoEConfig("mxfp8_small", 12, "mxfp8", 150, 512, 256, 16, 4, num_shared=1,
                             routing="sigmoid_normal"),
    "mxfp4_small": MoEConfig("mxfp4_small", 13, "mxfp4", 37, 512, 384, 32, 8, routing="softmax_uniform"),
    "nvfp4_small": MoEConfig("nvfp4_small", 14, "nvfp4", 300, 512, 256, 16, 6, routing="zipf"),
}

# More tiles than the persistent grid has workgroups, so each workgroup runs
# several tiles: with I = 1024 the next tile's first stages are prefetched
# during the current tile; with a short I (L2 K shorter than the copy ring)
# each tile fills the ring itself.  The short I is 256 for the MX formats:
# with I = 128 an L2 output sums only 128 products of coarse E2M1 / E4M3
# values, and one legitimate rounding-boundary flip of an MXFP8 L2 input
# (fp32 accumulation order vs float64) already moves it by a few percent of
# the output RMS.
SHORT_I = {"bf16": 128, "mxfp8": 256, "mxfp4": 256, "nvfp4": 128}
MULTI = {
    f"{fmt}_multi_i{inter}": MoEConfig(f"{fmt}_multi_i{inter}", 20 + 2 * i + j, fmt, 4000, 1024, inter, 8, 2,
                                       routing="softmax_uniform")
    for i, fmt in enumerate(["bf16", "mxfp8", "mxfp4", "nvfp4"]) for j, inter in enumerate([1024, SHORT_I[fmt]])
}

# BF16 layers whose L2 has more tiles than the grid has workgroups, with a
# partial last round that runs split in K parts (the split tail) while the
# other tiles run whole: 22 BLOCK_M-256 blocks x 16 column blocks = 352
# tiles, the last 96 in 2 parts of 8 stages; and x 24 column blocks = 528
# tiles, the last 16 in 4 parts of 2 stages each (too short to hand stages
# over to the next tile, so each part fills the copy ring itself).
TAIL = MoEConfig("bf16_tail", 60, "bf16", 2048, 4096, 512, 8, 2, routing="softmax_uniform")
TAIL_SHORT = MoEConfig("bf16_tail_short", 60, "bf16", 2048, 6144, 256, 8, 2, routing="softmax_uniform")
# the guard-band test also covers the split-tail L2's parts buffer and the
# many-workgroup dispatch (16384 slots) with its scale gather
GUARD_EXTRA = {
    "bf16_tail": TAIL,
    "mxfp8_many": MoEConfig("mxfp8_many", 70, "mxfp8", 2048, 512, 256, 64, 8, routing="softmax_uniform"),
    "nvfp4_many": MoEConfig("nvfp4_many", 71, "nvfp4", 2048, 512, 256, 64, 8, routing="zipf"),
}

_CACHE = {}


def inputs(cfg):
    if cfg.name not in _CACHE:
        x = bf16_bits(gen_x_bf16(cfg))
        ids, wts = gen_routing(cfg)
        _CACHE[cfg.name] = (x, ids, wts, make_weights(cfg))
    return _CACHE[cfg.name]


def l2_scale(cfg, factor=1.0):
    """NVFP4: the experts' w2 input scales (times ``factor``) and their max
    (1.0 if 0), the one global scale every L2 input is quantised with."""
    if cfg.fmt != "nvfp4":
        return None, 1.0
    w2in = (gen_w2_input_scale(cfg) * np.float32(factor)).astype(np.float32)
    m = float(w2in.max())
    return w2in, (m if m > 0 else 1.0)


def compare(cfg, block_m=0, act=None, w2in_scale=1.0, tag="", **kw):
    x, ids, wts, w = inputs(cfg)
    w2in, g2 = l2_scale(cfg, w2in_scale)
    y, _ = run_layer(cfg.fmt, x, ids, wts, w, num_shared=cfg.num_shared, block_m=block_m, act=act,
                     w2_input_scale=w2in, **kw)
    ref = moe_reference(cfg.fmt, x, ids, wts, w, num_shared=cfg.num_shared, act=act, l2_activation_scale=g2)
    rel, excess, alt = check_layer(cfg.fmt, y, ref, x, ids, wts, w, num_shared=cfg.num_shared, act=act, g2=g2,
                                   name=f"{cfg.name} bm={block_m}{tag}")
    print(f"{cfg.name} bm={block_m}: max|err|/RMS = {rel:.3e}, tokens under another valid L2-input decision: {alt}")
    assert excess <= 0, (rel, excess)
    assert alt <= rescue_cap(cfg.T), alt
    return y


@pytest.mark.parametrize("name", sorted(SMALL))
def test_forward_matches_oracle(name):
    compare(SMALL[name])


@pytest.mark.parametrize("bm", [32, 64, 128, 256])
@pytest.mark.parametrize("name", ["bf16_small", "mxfp8_small", "mxfp4_small", "nvfp4_small"])
def test_forward_every_block_m(name, bm):
    compare(SMALL[name], block_m=bm)


# Hidden 768: three 256-column N blocks in the L2 (an odd count) and six
# 128-K stages in the L1 (24 of 32 K for BF16), fewer than some rings hold
ODD_H = {f"{fmt}_h768": MoEConfig(f"{fmt}_h768", 70 + i, fmt, 120, 768, 384, 8, 2, routing="softmax_uniform")
         for i, fmt in enumerate(["bf16", "mxfp8", "mxfp4", "nvfp4"])}


@pytest.mark.parametrize("bm", [0, 64])
@pytest.mark.parametrize("name", sorted(ODD_H))
def test_forward_odd_hidden(name, bm):
    compare(ODD_H[name], block_m=bm)


@pytest.mark.parametrize("bm", [32, 128])
@pytest.mark.parametrize("name", sorted(MULTI))
def test_forward_several_tiles_per_workgroup(name, bm):
    compare(MULTI[name], block_m=bm)


@pytest.mark.parametrize("cfg,bm", [(TAIL, 0), (TAIL, 128), (TAIL_SHORT, 0)], ids=["bm0", "bm128", "short_parts"])
def test_forward_bf16_split_tail(cfg, bm):
    """The L2's partial last round split in K parts, the other tiles whole;
    the combine takes each slot's columns from the tile that computed them."""
    compare(cfg, block_m=bm)


def test_forward_bf16_split_tail_with_norm():
    """The post-expert RMSNorm combine over a split-tail L2."""
    cfg = TAIL
    x, ids, wts, w = inputs(cfg)
    gamma = np.random.default_rng(9).uniform(0.5, 1.5, cfg.H)
    norm = (gamma, 1e-6)
    y, _ = run_layer(cfg.fmt, x, ids, wts, w, norm=norm)
    pre = moe_reference(cfg.fmt, x, ids, wts, w)
    ref = moe_reference(cfg.fmt, x, ids, wts, w, norm=norm)
    rel, excess, alt = check_layer(cfg.fmt, y, ref, x, ids, wts, w, norm=norm, y_pre=pre)
    print(f"bf16_tail + norm: max|err|/RMS = {rel:.3e}")
    assert excess <= 0, (rel, excess)


@pytest.mark.parametrize("name", sorted(MULTI))
def test_forward_independent_of_block_m(name):
    """Every output element's K sums run in the same order whatever the tile
    height, so all BLOCK_M give bit-identical layers (a check of the tiling
    and the copy pipeline that needs no tolerance).  These layers have fewer
    L2 tiles than the grid has workgroups, so no split tail (whose split
    tiles depend on the tile height) applies."""
    cfg = MULTI[name]
    x, ids, wts, w = inputs(cfg)
    w2in, _ = l2_scale(cfg)
    ys = [run_layer(cfg.fmt, x, ids, wts, w, num_shared=cfg.num_shared, block_m=bm, w2_input_scale=w2in)[0]
          for bm in (32, 64, 128, 256)]
    for bm, y in zip((64, 128, 256), ys[1:]):
        assert np.array_equal(ys[0], y), bm


ACT_VARIANTS = [{"clamp": 0.75, "alpha": 1.702, "beta": 1.0}, {"clamp": None, "alpha": 0.5, "beta": -0.25},
                {"clamp": 0.0, "alpha": 1.0, "beta": 0.0}]


@pytest.mark.parametrize("name", ["bf16_small", "mxfp8_small", "mxfp4_small", "nvfp4_small", "bf16_decode",
                                  "mxfp8_decode", "mxfp4_decode", "nvfp4_decode"])
def test_forward_activation_variants(name):
    """MegaMoEActivation's clamp, alpha and beta in every format's L1
    epilogue, and in the finish kernel of a K-split L1 (decode-sized
    launches)."""
    cfg = {**SMALL, **DECODE_SMALL}[name]
    for i, act in enumerate(ACT_VARIANTS):
        compare(cfg, act=act, tag=f" act{i}")


@pytest.mark.parametrize("name", ["nvfp4_small", "nvfp4_decode"])
def test_forward_nvfp4_saturated_l2_input(name):
    """An NVFP4 L2 input scale 64 times below the calibrated one: many L2
    input block scales clamp at 448 and elements at 6, in the L1 epilogue and
    in the K-split finish kernel; the oracle applies the same scale."""
    compare({**SMALL, **DECODE_SMALL}[name], w2in_scale=1.0 / 64, tag=" saturated")


@pytest.mark.parametrize("name", ["bf16_small", "mxfp8_small", "mxfp4_small", "nvfp4_small", "mxfp4_decode",
                                  *GUARD_EXTRA])
def test_forward_writes_nothing_outside_out_and_workspace(name):
    """Guard bands of a known pattern around ``out`` and the workspace are
    untouched by a forward, and every element of ``out`` is written."""
    from expert_gemms_amd import _lib
    cfg = {**SMALL, **DECODE_SMALL, **GUARD_EXTRA}[name]
    x, ids, wts, w = inputs(cfg)
    w2in, _ = l2_scale(cfg)
    _, layer = run_layer(cfg.fmt, x, ids, wts, w, num_shared=cfg.num_shared, w2_input_scale=w2in)
    G = 1 << 16                                          # guard bytes on each side
    n_out = cfg.T * cfg.H * 2
    out_buf = torch.full((G + n_out + G,), 0x5A, dtype=torch.uint8, device="cuda")
    out_buf[G:G + n_out] = 0xFF                          # BF16 NaNs until written
    out = out_buf[G:G + n_out].view(torch.bfloat16).view(cfg.T, cfg.H)
    nws = layer.workspace.numel()
    ws_buf = torch.full((G + nws + G,), 0xA5, dtype=torch.uint8, device="cuda")
    ws = ws_buf[G:G + nws]
    _lib.moe_forward(cfg.fmt, cfg.T, cfg.H, cfg.I, cfg.top_k, 0, cfg.E, cfg.num_shared, 0, None, x_dev(x),
                     dev(ids.astype(np.int32)), dev(wts.astype(np.float32)), layer.w13_k, layer.w13_sf_k,
                     layer.w2_k, layer.w2_sf_k, layer.w13_gs, layer.w2_gs, layer.l2_activation_scale, out, ws)
    torch.cuda.synchronize()
    ob, wb = out_buf.cpu().numpy(), ws_buf.cpu().numpy()
    assert (ob[:G] == 0x5A).all() and (ob[G + n_out:] == 0x5A).all()
    assert (wb[:G] == 0xA5).all() and (wb[G + nws:] == 0xA5).all()
    assert torch.isfinite(out.float()).all()


def test_forward_expert_range_and_dropped_slots():
    """A GPU holding experts 2..5 of 8: other ids (and -1) drop their slots."""
    cfg = SMALL["bf16_small"]
    x, ids, wts, w = inputs(cfg)
    ids = ids.copy()
    ids[::7, 1] = -1
    w_loc = {k: v[2:6] for k, v in w.items()}
    y, _ = run_layer("bf16", x, ids, wts, w_loc, expert_start=2, num_local=4)
    ref = moe_reference("bf16", x, ids, wts, w_loc, expert_start=2, num_local=4)
    rel, excess = check_output("bf16", y, ref)
    assert excess <= 0, rel
    none_local = ~np.isin(ids, [2, 3, 4, 5]).any(axis=1)
    assert none_local.any() and not y[none_local].any()      # such tokens get zeros


def test_forward_all_dropped_and_single_token():
    cfg = SMALL["mxfp8_small"]
    x, ids, wts, w = inputs(cfg)
    w_r = {k: v[:cfg.E] for k, v in w.items()}
    y, _ = run_layer("mxfp8", x, np.full_like(ids, -1), wts, w_r)
    assert not y.any()
    y1, _ = run_layer("mxfp8", x[:1], ids[:1], wts[:1], w_r)
    ref1 = moe_reference("mxfp8", x[:1], ids[:1], wts[:1], w_r)
    assert check_layer("mxfp8", y1, ref1, x[:1], ids[:1], wts[:1], w_r)[1] <= 0


@pytest.mark.parametrize("name", ["mxfp8_small", "nvfp4_small"])
def test_forward_deterministic(name):
    cfg = SMALL[name]
    x, ids, wts, w = inputs(cfg)
    w2in, _ = l2_scale(cfg)
    a, _ = run_layer(cfg.fmt, x, ids, wts, w, num_shared=cfg.num_shared, w2_input_scale=w2in)
    b, _ = run_layer(cfg.fmt, x, ids, wts, w, num_shared=cfg.num_shared, w2_input_scale=w2in)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["bf16_small", "mxfp8_small", "mxfp4_small", "nvfp4_small"])
def test_forward_post_expert_norm(name):
    """Post-expert RMSNorm fused into the combine (Muse-Spark MegaMoE page)."""
    cfg = SMALL[name]
    x, ids, wts, w = inputs(cfg)
    w2in, g2 = l2_scale(cfg)
    gamma = np.random.default_rng(7).uniform(0.5, 1.5, cfg.H)
    norm = (gamma, 1e-6)
    y, _ = run_layer(cfg.fmt, x, ids, wts, w, num_shared=cfg.num_shared, w2_input_scale=w2in, norm=norm)
    pre = moe_reference(cfg.fmt, x, ids, wts, w, num_shared=cfg.num_shared, l2_activation_scale=g2)
    ref = moe_reference(cfg.fmt, x, ids, wts, w, num_shared=cfg.num_shared, l2_activation_scale=g2, norm=norm)
    rel, excess, alt = check_layer(cfg.fmt, y, ref, x, ids, wts, w, num_shared=cfg.num_shared, g2=g2, norm=norm,
                                   y_pre=pre)
    print(f"{name} + norm: max|err|/RMS = {rel:.3e}, tokens under another valid decision: {alt}")
    assert excess <= 0, (rel, excess)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp8", "mxfp4", "nvfp4"])
def test_forward_router_weight_on_input(fmt):
    """apply_router_weight_on_input (top_k = 1, no shared expert)."""
    from oracle.moe import weight_on_input
    cfg = MoEConfig(f"woi_{fmt}", 50, fmt, 300, 512, 256, 8, 1, routing="softmax_uniform")
    x, ids, wts, w = inputs(cfg)
    wts = np.random.default_rng(8).uniform(0.2, 1.0, ids.shape).astype(np.float32)
    w2in, g2 = l2_scale(cfg)
    y, _ = run_layer(fmt, x, ids, wts, w, w2_input_scale=w2in, weight_on_input=True)
    ref = moe_reference(fmt, x, ids, wts, w, l2_activation_scale=g2, router_weight_on_input=True)
    rel, excess, alt = check_layer(fmt, y, ref, weight_on_input(x, wts), ids, np.ones_like(wts), w, g2=g2)
    print(f"{fmt} weight on input: max|err|/RMS = {rel:.3e}, tokens under another valid decision: {alt}")
    assert excess <= 0, (rel, excess)


@pytest.mark.parametrize("name", ["nvfp4_small", "mxfp8_multi_i1024"])
def test_forward_graph_replay(name):
    """One forward captured in a HIP graph and replayed three times, with
    eager forwards of other inputs on the same workspace in between: every
    replay equals the eager result bit for bit (no step reads workspace left
    by an earlier call)."""
    from tests.gpu_util import dev, x_dev
    cfg = {**SMALL, **MULTI}[name]
    x, ids, wts, w = inputs(cfg)
    w2in, _ = l2_scale(cfg)
    _, layer = run_layer(cfg.fmt, x, ids, wts, w, num_shared=cfg.num_shared, w2_input_scale=w2in)
    xd, idd, wd = x_dev(x), dev(ids.astype(np.int32)), dev(wts.astype(np.float32))
    eager = layer.forward(xd, idd, wd).clone()
    # other inputs: the tokens reversed and fewer of them
    T2 = max(1, cfg.T // 2)
    x2, id2, w2 = x_dev(x[::-1][:T2]), dev(ids[::-1][:T2].astype(np.int32)), dev(wts[::-1][:T2].astype(np.float32))
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(xd, idd, wd, out=out)          # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(xd, idd, wd, out=out)
    for i in range(3):
        out.zero_()
        other = layer.forward(x2, id2, w2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        assert other.abs().sum() > 0


def test_forward_norm_zero_centred_gain_folded_by_holder():
    """set_post_expert_norm(weight, eps, gain_center) ≡ passing gamma =
    weight + gain_center to forward, bit for bit."""
    from tests.gpu_util import dev, x_dev
    cfg = SMALL["bf16_small"]
    x, ids, wts, w = inputs(cfg)
    _, layer = run_layer(cfg.fmt, x, ids, wts, w)
    gamma = torch.from_numpy(np.random.default_rng(7).uniform(0.5, 1.5, cfg.H).astype(np.float32))
    xd, idd, wd = x_dev(x), dev(ids.astype(np.int32)), dev(wts.astype(np.float32))
    direct = layer.forward(xd, idd, wd, norm_gamma=gamma.cuda(), norm_eps=1e-6)
    layer.set_post_expert_norm(gamma - 1.0, 1e-6, gain_center=1.0)
    folded = layer.forward(xd, idd, wd)
    torch.cuda.synchronize()
    # gamma - 1 + 1 may differ from gamma in its last bit; compare against that gamma
    g2 = (gamma - 1.0) + 1.0
    again = layer.forward(xd, idd, wd, norm_gamma=g2.cuda(), norm_eps=1e-6)
    assert torch.equal(folded, again)
    assert torch.allclose(folded.float(), direct.float(), rtol=1e-2, atol=1e-2)


# Decode-sized launches: few tiles, so the L1 GEMM's K is split into parts
# summed by the finish kernel before the activation.
DECODE_SMALL = {
    f"{fmt}_decode": MoEConfig(f"{fmt}_decode", 60 + i, fmt, 3, 512, 256, 32, 4, routing="softmax_uniform")
    for i, fmt in enumerate(["bf16", "mxfp8", "mxfp4", "nvfp4"])
}


@pytest.mark.parametrize("name", sorted(DECODE_SMALL))
def test_forward_decode_split_l1(name):
    cfg = DECODE_SMALL[name]
    ys = [compare(cfg, block_m=bm) for bm in (32, 64, 128, 256)]
    for bm, y in zip((64, 128, 256), ys[1:]):
        assert np.array_equal(ys[0], y), bm
