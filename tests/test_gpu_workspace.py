"""What the forward itself computed, read back from its workspace
(moe_workspace_layout): the routing metadata and the dispatch-quantised x
bit-exact against the oracle (whichever dispatch kernel the forward took:
the single-workgroup dispatch fused with the MX quantisation below 16384
slots, the three-launch dispatch above), and the L2-input codes and block
scales (a5) against the oracle's quantiser applied to the oracle's
activations, where a code may differ only at a decision boundary within the
GPU's evaluation error (tests/helpers.l2_code_check; for the MX formats that
error includes the scaled MFMA's own, see tests/helpers.MX_MFMA_STEP_BOUND),
and, with inputs whose L1 sums are exact on the GPU, code for code.
"""

import numpy as np
import pytest

from oracle import codecs, quant
from oracle.dispatch import dispatch_reference
from synth import MoEConfig, gen_routing, gen_x_bf16, gen_w2_input_scale, bf16_bits
from tests.gpu_util import WorkspaceReader, run_layer
from tests.helpers import l2_code_check, make_weights, record_parity, slot_l2_inputs

pytestmark = pytest.mark.gpu

CASES = {
    # MX below 16384 slots: dispatch and x quantisation in one launch
    "mxfp8_shared": MoEConfig("ws_mxfp8_shared", 80, "mxfp8", 150, 512, 256, 16, 4, num_shared=1,
                              routing="sigmoid_normal"),
    "mxfp4_decode": MoEConfig("ws_mxfp4_decode", 81, "mxfp4", 3, 512, 256, 32, 4, routing="softmax_uniform"),
    "mxfp4_multi": MoEConfig("ws_mxfp4_multi", 82, "mxfp4", 1500, 1024, 256, 8, 2, routing="softmax_uniform"),
    # MX from 16384 slots on: the three-launch dispatch and a separate quantisation
    "mxfp8_many": MoEConfig("ws_mxfp8_many", 83, "mxfp8", 2100, 256, 256, 16, 8, routing="softmax_normal"),
    "nvfp4_zipf": MoEConfig("ws_nvfp4_zipf", 84, "nvfp4", 300, 512, 256, 16, 6, routing="zipf"),
    "nvfp4_decode": MoEConfig("ws_nvfp4_decode", 85, "nvfp4", 3, 512, 256, 32, 4, routing="softmax_uniform"),
    "bf16": MoEConfig("ws_bf16", 86, "bf16", 200, 512, 384, 8, 2, routing="softmax_uniform"),
    "bf16_decode": MoEConfig("ws_bf16_decode", 87, "bf16", 3, 512, 256, 32, 4, routing="softmax_uniform"),
}

_CACHE = {}


def inputs(cfg):
    if cfg.name not in _CACHE:
        x = bf16_bits(gen_x_bf16(cfg))
        ids, wts = gen_routing(cfg)
        _CACHE[cfg.name] = (x, ids, wts, make_weights(cfg))
    return _CACHE[cfg.name]


def forward(cfg, block_m=0, act=None, w2in_scale=1.0):
    x, ids, wts, w = inputs(cfg)
    w2in = gen_w2_input_scale(cfg) * np.float32(w2in_scale) if cfg.fmt == "nvfp4" else None
    y, layer = run_layer(cfg.fmt, x, ids, wts, w, num_shared=cfg.num_shared, block_m=block_m, act=act,
                         w2_input_scale=w2in)
    return y, layer, WorkspaceReader(layer, cfg.T, block_m)


@pytest.mark.parametrize("bm", [0, 32, 128])
@pytest.mark.parametrize("name", sorted(CASES))
def test_dispatch_and_quantised_x_from_the_forward(name, bm):
    cfg = CASES[name]
    x, ids, _, _ = inputs(cfg)
    _, _, ws = forward(cfg, block_m=bm)
    ref = dispatch_reference(ids, cfg.num_shared, 0, cfg.E, ws.bm)
    got = ws.dispatch()
    for k in ref:
        assert np.array_equal(got[k], ref[k]), k
    if cfg.fmt == "bf16":
        return
    x32 = codecs.bf16_decode(x).astype(np.float32)
    codes, scales, tok = ws.xq()
    if cfg.fmt == "nvfp4":
        g = quant.nvfp4_global_scale(np.abs(x32).max(axis=1))
        q, bs = quant.nvfp4_quantize(x32, g)
        assert np.array_equal(tok, g)
        fill = 0x38                                  # E4M3 1.0
    else:
        q, bs = quant.mx_quantize(x32, "e4m3")
        fill = 127                                   # UE8M0 1.0
    assert np.array_equal(codes, q)
    assert np.array_equal(scales, bs)
    # the scales the L1 GEMM reads: each sorted row's token's, padding rows 1.0
    M = int(ref["offsets"][-1])
    planes = ws.a1_planes(M)
    ss = ref["sorted_slot"]
    real = ss >= 0
    kk = cfg.top_k + cfg.num_shared
    assert np.array_equal(planes[real], bs[ss[real] // kk])
    assert (planes[~real] == fill).all()


L2_CASES = [("mxfp8_shared", 0), ("mxfp8_shared", 32), ("mxfp4_decode", 0), ("mxfp4_multi", 128),
            ("mxfp8_many", 0), ("nvfp4_zipf", 0), ("nvfp4_zipf", 128), ("nvfp4_decode", 0), ("bf16", 0),
            ("bf16", 256), ("bf16_decode", 0)]


def l2_check(name, bm, act=None, w2in_scale=1.0, tag=""):
    cfg = CASES[name]
    x, ids, _, w = inputs(cfg)
    _, layer, ws = forward(cfg, block_m=bm, act=act, w2in_scale=w2in_scale)
    slots, _, a, da = slot_l2_inputs(cfg.fmt, x, ids, w, num_shared=cfg.num_shared, act=act)
    rows = ws.dispatch()["slot_row"][slots]
    assert (rows >= 0).all()
    codes, scales = ws.l2_input(rows)
    st = l2_code_check(cfg.fmt, codes, scales, a, da, g2=layer.l2_activation_scale)
    record_parity(f"L2 input {name}{tag} bm={ws.bm} (L1 split {ws.lay['l1_ksplit']})", **st)
    assert st["unexplained"] == 0, st
    # boundary cases are rare: a systematic slip would flip far more codes
    # (the MX formats' wider evaluation error leaves more of them)
    cap = 5e-3 if cfg.fmt in ("mxfp8", "mxfp4") else 1e-3
    assert st["element_flips"] <= max(2, cap * st["elements"]), st
    assert st["scale_flips"] <= max(2, 1e-2 * st["blocks"]), st
    return st, ws, a


@pytest.mark.parametrize("name,bm", L2_CASES, ids=[f"{n}-bm{b}" for n, b in L2_CASES])
def test_l2_input_codes_match_the_oracle_quantiser(name, bm):
    l2_check(name, bm)


@pytest.mark.parametrize("name", ["mxfp8_shared", "mxfp4_decode", "nvfp4_zipf", "nvfp4_decode", "bf16_decode"])
def test_l2_input_codes_under_activation_variants(name):
    l2_check(name, 0, act={"clamp": 0.75, "alpha": 1.702, "beta": 1.0}, tag=" clamp/alpha/beta")


@pytest.mark.parametrize("name", ["nvfp4_zipf", "nvfp4_decode"])
def test_l2_input_codes_when_nvfp4_block_scales_saturate(name):
    """An L2 input scale far below the activations' (a checkpoint calibrated
    on other data): block scales clamp at E4M3 448 and elements at E2M1 6."""
    st, ws, a = l2_check(name, 0, w2in_scale=1.0 / 64, tag=" saturated")
    _, scales = ws.l2_input(ws.dispatch()["slot_row"][ws.dispatch()["slot_row"] >= 0])
    assert (scales == 0x7E).any()                    # some block scale saturated at 448


# ---------------------------------------------------------------------------
# Exact L1 sums: x in {-2, -1, 1, 2} and weights in {-1.5, -1, 1, 1.5} * 2^-5
# quantise without loss in every format (NVFP4 up to its float32 scales),
# every product has at most two significant bits within two binades, and
# every sum is exact in float32, in the scaled MFMA (exact for products this
# narrow) and across K-split parts.  The GPU's g and u then equal the
# oracle's (NVFP4: up to its two float32 scale products), so each L2-input
# code must be the oracle's except where the hardware exp / reciprocal
# (2^-18) straddles a decision: this pins the epilogue's quantiser (scale
# choice, rounding, saturation, packing) code for code, unsplit and split.
EXACT = {
    "many": dict(T=2000, H=1024, I=1024, E=8, k=2),     # unsplit L1 epilogue
    "decode": dict(T=3, H=512, I=256, E=32, k=4),       # K-split L1 + finish kernel
}


def exact_inputs(fmt, shape, seed):
    from synth import MoEConfig
    from tests.helpers import quantize_weight
    rng = np.random.default_rng(seed)
    T, H, I, E, k = (shape[n] for n in ("T", "H", "I", "E", "k"))
    x32 = rng.choice(np.array([-2.0, -1.0, 1.0, 2.0], np.float32), (T, H))
    x = codecs.bf16_encode_f32(x32)
    cfg = MoEConfig(f"exact_{fmt}_{T}", seed, fmt, T, H, I, E, k, routing="softmax_uniform")
    ids, wts = gen_routing(cfg)
    grid = np.array([-1.5, -1.0, 1.0, 1.5], np.float32) * np.float32(2.0 ** -5)
    parts = {nm: [quantize_weight(fmt, rng.choice(grid, shp)) for _ in range(E)]
             for nm, shp in (("w13", (2 * I, H)), ("w2", (H, I)))}
    w = {}
    for nm, ps in parts.items():
        w[nm] = np.stack([p["w"] for p in ps])
        if "sf" in ps[0]:
            w[nm + "_sf"] = np.stack([p["sf"] for p in ps])
        if "gs" in ps[0]:
            w[nm + "_gs"] = np.array([p["gs"] for p in ps], dtype=np.float32)
    return x, ids, wts, w


@pytest.mark.parametrize("act", [None, {"clamp": 7.0, "alpha": 1.702, "beta": 1.0}], ids=["swiglu", "variant"])
@pytest.mark.parametrize("fmt", ["bf16", "mxfp8", "mxfp4", "nvfp4"])
def test_l2_input_codes_with_exact_l1_sums(fmt, act):
    splits = {}
    for name, shape in EXACT.items():
        x, ids, wts, w = exact_inputs(fmt, shape, 500 + len(name))
        w2in = np.full(shape["E"], 16.0 / 2688.0, np.float32) if fmt == "nvfp4" else None
        _, layer = run_layer(fmt, x, ids, wts, w, act=act, w2_input_scale=w2in)
        ws = WorkspaceReader(layer, shape["T"])
        splits[name] = ws.lay["l1_ksplit"]
        slots, _, a, da = slot_l2_inputs(fmt, x, ids, w, act=act, exact=True)
        codes, scales = ws.l2_input(ws.dispatch()["slot_row"][slots])
        st = l2_code_check(fmt, codes, scales, a, da, g2=layer.l2_activation_scale)
        record_parity(f"L2 input exact sums {fmt} {name}{'' if act is None else ' variant'} "
                      f"(L1 split {splits[name]})", **st)
        assert st["unexplained"] == 0, st
        assert st["element_flips"] + st["scale_flips"] <= max(2, 1e-4 * st["elements"]), st
    assert splits["many"] == 1 and splits["decode"] > 1, splits     # both epilogues covered
