"""Pins of the oracle's layer function ``moe_reference``.

* top_k = 1 with weight 1 equals a dense gated MLP per token, computed here
  by a different route: all experts for all tokens with torch float64
  einsums and torch's silu, weights dequantised through torch's own float8
  views, then the token's expert selected.
* invariance under expert relabelling; zero-weight slots contribute nothing;
  linearity in the routing weights; x = 0 gives y = 0;
* a fused shared expert equals the routed output plus a dense MLP;
* non-local expert ids are dropped; a token subset equals the full rows;
* scalar-loop brute force on tiny shapes for every format;
* swiglu's clamp / alpha / beta closed forms.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import codecs, quant
from oracle import moe as M
from synth import MoEConfig, gen_x_bf16, gen_routing, bf16_bits
from tests.helpers import make_weights

GOLD = os.path.join(os.path.dirname(__file__), "golden")
_E2M1 = None


def _e2m1_table():
    global _E2M1
    if _E2M1 is None:
        with open(os.path.join(GOLD, "e2m1_values.json")) as f:
            g = json.load(f)["code_to_value"]
        _E2M1 = torch.tensor([g[str(i)] for i in range(16)], dtype=torch.float64)
    return _E2M1


def torch_dequant(fmt, w, name):
    """Independent dequantisation: torch float8 views and the golden E2M1
    table, float64 [E, N, K]."""
    a = torch.from_numpy(np.ascontiguousarray(w[name]))
    if fmt == "bf16":
        return a.view(torch.int16).view(torch.bfloat16).double()
    if fmt == "mxfp8":
        v = a.view(torch.float8_e4m3fn).double()
    else:
        lo, hi = (a & 0xF).long(), (a >> 4).long()
        v = torch.stack([_e2m1_table()[lo], _e2m1_table()[hi]], -1).flatten(-2)
    K = v.shape[-1]
    if fmt in ("mxfp8", "mxfp4"):
        sf = torch.from_numpy(w[name + "_sf"]).long()
        s = torch.ldexp(torch.ones_like(sf, dtype=torch.float64), sf - 127)
        s = torch.where(sf == 0, torch.zeros_like(s), s)
        return (v.view(*v.shape[:-1], K // 32, 32) * s[..., None]).view(v.shape)
    bs = torch.from_numpy(w[name + "_sf"]).view(torch.float8_e4m3fn).double()
    gs = torch.from_numpy(w[name + "_gs"]).double()
    return (v.view(*v.shape[:-1], K // 16, 16) * bs[..., None]).view(v.shape) * gs[:, None, None]


def torch_x(fmt, x_bits):
    """Dispatch-quantised x through the oracle's (separately pinned)
    quantisers, but assembled independently of moe_reference."""
    x32 = torch.from_numpy(x_bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    if fmt == "bf16":
        return torch.from_numpy(x32).double()
    if fmt in ("mxfp8", "mxfp4"):
        q, c = quant.mx_quantize(x32, "e4m3")
        v = torch.from_numpy(q).view(torch.float8_e4m3fn).double()
        s = torch.from_numpy(codecs.ue8m0_decode(c))
        return (v.view(v.shape[0], -1, 32) * s[..., None]).view(v.shape)
    g = quant.nvfp4_global_scale(np.abs(x32).max(axis=1))
    q, bs = quant.nvfp4_quantize(x32, g)
    v = _e2m1_table()[torch.from_numpy(q).long()]
    b = torch.from_numpy(bs).view(torch.float8_e4m3fn).double()
    return (v.view(v.shape[0], -1, 16) * b[..., None]).view(v.shape) * torch.from_numpy(g).double()[:, None]


def torch_l2q(fmt, a, g2):
    a32 = a.float()
    if fmt == "bf16":
        return a32.bfloat16().double()
    n = a32.shape[:-1]
    flat = a32.reshape(-1, a32.shape[-1]).numpy()
    if fmt in ("mxfp8", "mxfp4"):
        q, c = quant.mx_quantize(flat, "e4m3")
        v = torch.from_numpy(q).view(torch.float8_e4m3fn).double()
        s = torch.from_numpy(codecs.ue8m0_decode(c))
        out = (v.view(v.shape[0], -1, 32) * s[..., None]).view(v.shape)
    else:
        g = np.full(flat.shape[0], np.float32(g2))
        q, bs = quant.nvfp4_quantize(flat, g)
        v = _e2m1_table()[torch.from_numpy(q).long()]
        b = torch.from_numpy(bs).view(torch.float8_e4m3fn).double()
        out = (v.view(v.shape[0], -1, 16) * b[..., None]).view(v.shape) * float(np.float32(g2))
    return out.view(*n, -1)


def dense_top1(fmt, x_bits, ids, w, g2=1.0):
    X = torch_x(fmt, x_bits)                                   # [T, H]
    W13 = torch_dequant(fmt, w, "w13")                         # [E, 2I, H]
    W2 = torch_dequant(fmt, w, "w2")                           # [E, H, I]
    I = W13.shape[1] // 2
    G = torch.einsum("th,eih->tei", X, W13[:, :I])
    U = torch.einsum("th,eih->tei", X, W13[:, I:])
    A = torch.nn.functional.silu(G) * U
    A = torch_l2q(fmt, A, g2)
    O = torch.einsum("tei,ehi->teh", A, W2)
    return O[torch.arange(X.shape[0]), torch.from_numpy(ids[:, 0]).long()].numpy()


def small_cfg(fmt, T=24, H=64, I=64, E=5, k=2, n_sh=0, routing="softmax_normal", cid=91):
    return MoEConfig(f"pin_{fmt}", cid, fmt, T, H, I, E, k, n_sh, routing)


FMTS = ["bf16", "mxfp8", "mxfp4", "nvfp4"]


@pytest.mark.parametrize("fmt", FMTS)
def test_top1_weight1_equals_dense_gated_mlp(fmt):
    cfg = small_cfg(fmt, k=1)
    x = bf16_bits(gen_x_bf16(cfg))
    ids, _ = gen_routing(cfg)
    w = make_weights(cfg)
    g2 = 0.013
    y = M.moe_reference(fmt, x, ids, np.ones(ids.shape, np.float32), w, l2_activation_scale=g2)
    ref = dense_top1(fmt, x, ids, w, g2)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("fmt", FMTS)
def test_relabelling_invariance(fmt):
    cfg = small_cfg(fmt, k=3, n_sh=1)
    x = bf16_bits(gen_x_bf16(cfg))
    ids, wts = gen_routing(cfg)
    w = make_weights(cfg)
    y = M.moe_reference(fmt, x, ids, wts, w, num_shared=1)
    perm = np.random.default_rng(5).permutation(cfg.E)        # routed experts only
    inv = np.argsort(perm)
    full = np.concatenate([inv, [cfg.E]])                      # new expert p holds old inv[p]
    w2 = {k: v[full] for k, v in w.items()}
    y2 = M.moe_reference(fmt, x, perm[ids].astype(np.int32), wts, w2, num_shared=1)
    assert np.allclose(y, y2, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_zero_weight_slot_is_a_dropped_slot_and_linearity():
    cfg = small_cfg("mxfp8", k=3)
    x = bf16_bits(gen_x_bf16(cfg))
    ids, wts = gen_routing(cfg)
    w = make_weights(cfg)
    wz = wts.copy()
    wz[:, 1] = 0
    idz = ids.copy()
    idz[:, 1] = -1
    a = M.moe_reference("mxfp8", x, ids, wz, w)
    b = M.moe_reference("mxfp8", x, idz, wts, w)
    assert np.array_equal(a, b)
    y = M.moe_reference("mxfp8", x, ids, wts, w)
    y4 = M.moe_reference("mxfp8", x, ids, wts * np.float32(4.0), w)
    assert np.array_equal(4.0 * y, y4)


def test_zero_input_gives_zero_output():
    cfg = small_cfg("nvfp4", n_sh=1)
    ids, wts = gen_routing(cfg)
    w = make_weights(cfg)
    x = np.zeros((cfg.T, cfg.H), dtype=np.uint16)
    assert not M.moe_reference("nvfp4", x, ids, wts, w, num_shared=1).any()


@pytest.mark.parametrize("fmt", ["bf16", "mxfp8"])
def test_shared_expert_is_routed_plus_dense(fmt):
    cfg = small_cfg(fmt, k=2, n_sh=1)
    x = bf16_bits(gen_x_bf16(cfg))
    ids, wts = gen_routing(cfg)
    w = make_weights(cfg)
    y = M.moe_reference(fmt, x, ids, wts, w, num_shared=1)
    w_routed = {k: v[:cfg.E] for k, v in w.items()}
    y_routed = M.moe_reference(fmt, x, ids, wts, w_routed)
    w_sh = {k: v[cfg.E:] for k, v in w.items()}
    dense = dense_top1(fmt, x, np.zeros((cfg.T, 1), np.int32), w_sh)
    assert np.allclose(y, y_routed + dense, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_nonlocal_ids_dropped_and_token_subset():
    cfg = small_cfg("bf16", k=2, E=8)
    x = bf16_bits(gen_x_bf16(cfg))
    ids, wts = gen_routing(cfg)
    w = make_weights(cfg)
    # a rank owning experts 2..5 sees weights of those experts only
    w_loc = {k: v[2:6] for k, v in w.items()}
    y_loc = M.moe_reference("bf16", x, ids, wts, w_loc, expert_start=2, num_local=4)
    ids_m = np.where((ids >= 2) & (ids < 6), ids, -1).astype(np.int32)
    y_all = M.moe_reference("bf16", x, ids_m, wts, w)
    assert np.allclose(y_loc, y_all, rtol=1e-13, atol=1e-13)
    sub = [3, 0, 17]
    ys = M.moe_reference("bf16", x, ids, wts, w, tokens=sub)
    yf = M.moe_reference("bf16", x, ids, wts, w)
    assert np.allclose(ys, yf[sub], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("fmt", FMTS)
def test_scalar_bruteforce_tiny(fmt):
    cfg = small_cfg(fmt, T=3, H=32, I=32, E=3, k=2, n_sh=1, cid=93)
    x = bf16_bits(gen_x_bf16(cfg))
    ids, wts = gen_routing(cfg)
    ids[1, 1] = ids[1, 0]                                      # duplicate choice
    w = make_weights(cfg)
    g2 = 0.02
    y = M.moe_reference(fmt, x, ids, wts, w, num_shared=1, l2_activation_scale=g2)
    X = torch_x(fmt, x).tolist()
    W13 = torch_dequant(fmt, w, "w13").tolist()
    W2 = torch_dequant(fmt, w, "w2").tolist()
    I, H = cfg.I, cfg.H
    out = [[0.0] * H for _ in range(cfg.T)]
    for t in range(cfg.T):
        slots = [(int(ids[t, j]), float(wts[t, j])) for j in range(2)] + [(cfg.E, 1.0)]
        for e, wt in slots:
            a = []
            for i in range(I):
                g = sum(W13[e][i][h] * X[t][h] for h in range(H))
                u = sum(W13[e][I + i][h] * X[t][h] for h in range(H))
                a.append(g / (1.0 + math.exp(-g)) * u)
            ah = torch_l2q(fmt, torch.tensor([a], dtype=torch.float64), g2)[0].tolist()
            for h in range(H):
                out[t][h] += wt * sum(W2[e][h][i] * ah[i] for i in range(I))
    assert np.allclose(y, np.array(out), rtol=1e-11, atol=1e-12)


def test_activation_variants_closed_forms():
    rng = np.random.default_rng(7)
    g, u = rng.standard_normal((2, 1000)) * 4
    silu = torch.nn.functional.silu(torch.from_numpy(g)).numpy()
    assert np.allclose(M.activation(g, u), silu * u, rtol=1e-14)
    assert np.array_equal(M.activation(g, u, clamp=np.inf), M.activation(g, u))
    c = 1.5
    ref = np.minimum(g, c) / (1 + np.exp(-1.702 * np.minimum(g, c))) * (np.clip(u, -c, c) + 1.0)
    assert np.allclose(M.activation(g, u, clamp=c, alpha=1.702, beta=1.0), ref, rtol=1e-14)


@pytest.mark.parametrize("fmt", FMTS)
def test_slot_activations_equal_the_dense_route(fmt):
    """slot_activations (the values entering the L2-input quantiser) equal
    silu(G) * U of the dense torch route, picked at each slot's expert, for
    every slot of a top-2 routing with a shared expert."""
    cfg = small_cfg(fmt, T=20, E=5, k=2, n_sh=1, cid=97)
    x = bf16_bits(gen_x_bf16(cfg))
    ids, _ = gen_routing(cfg)
    ids = ids.copy()
    ids[3, 1] = -1                                              # a dropped slot has no activation
    w = make_weights(cfg)
    slots, experts, a = M.slot_activations(fmt, x, ids, w, num_shared=1)
    X = torch_x(fmt, x)
    W13 = torch_dequant(fmt, w, "w13")
    I = W13.shape[1] // 2
    G = torch.einsum("th,eih->tei", X, W13[:, :I])
    U = torch.einsum("th,eih->tei", X, W13[:, I:])
    A = (torch.nn.functional.silu(G) * U).numpy()
    kk = 3
    assert slots.size == 20 * kk - 1 and 3 * kk + 1 not in set(slots.tolist())
    for s, e, row in zip(slots, experts, a):
        t, j = divmod(int(s), kk)
        assert e == (ids[t, j] if j < 2 else 5)
        np.testing.assert_allclose(row, A[t, e], rtol=1e-12, atol=1e-14)
    # restricted to some tokens: the same rows
    s2, _, a2 = M.slot_activations(fmt, x, ids, w, num_shared=1, tokens=[4, 11])
    for s, row in zip(s2, a2):
        np.testing.assert_allclose(row, a[list(slots).index(s)], rtol=1e-12, atol=1e-15)
