"""The fused MoE routed-expert layer, written out plainly (oracle side).

What is computed follows the "DeepGEMM MegaMoE experts" page:

* ``DeepGemmMegaMoEExperts.forward``: BF16 hidden states [T, H], routing
  weights and logical expert ids [T, top_k] in, BF16 [T, H] out, routed plus
  (fused) shared expert output.
* ``_create_weights``: w13 is [E, 2I, H] (gate rows first, then up rows, as
  the "fused_moe" page's ``FusedMoE.weight_loader`` fills the two halves),
  w2 is [E, H, I]; a fused shared expert has the layout of one routed expert
  slice and is always selected.
* ``MegaMoEActivation``: swiglu is ``gate * sigmoid(alpha * gate) * (up +
  beta)`` after clamping gate from above and up on both sides to ``clamp``.
* module docstring and class docstring: MX weights and activations use UE8M0
  scales per 1x32; NVFP4 weights use E4M3 per 1x16 and a per-expert FP32
  global scale, dispatch uses a per-token FP32 scale, and every L2 input is
  quantised with one scale (the max of the experts' L2 input scales).

and the step order of the "fused_moe" page's ``DeepGemmExperts.apply``
(dispatch-quantised input, first grouped GEMM, activation, quantisation of
the L2 input, second grouped GEMM, weighted reduction by token).

Per token t and slot j (routed expert ``topk_ids[t, j]`` with weight
``topk_weights[t, j]``; shared experts with weight 1):

    x_hat = Deq(Q_x(x_t))                 dispatch quantisation (BF16: none)
    [g; u] = Deq(W13_e) @ x_hat           float64
    a      = act(g, u)                    float64
    a_hat  = Deq(Q_a(float32(a)))         L2-input quantisation
    o      = Deq(W2_e) @ a_hat            float64
    y_t    = sum_j w_tj * o               float64 (not rounded to BF16 here)

Formats and their canonical (untransformed) weight arrays, all NumPy:

    "bf16":  w13 uint16 bits [E, 2I, H]; w2 uint16 bits [E, H, I]
    "mxfp8": w13 uint8 E4M3 [E, 2I, H] + w13_sf uint8 UE8M0 [E, 2I, H/32];
             w2 [E, H, I] + w2_sf [E, H, I/32]; activations MXFP8
    "mxfp4": w13 uint8 packed E2M1 [E, 2I, H/2] + w13_sf UE8M0 [E, 2I, H/32];
             w2 [E, H, I/2] + w2_sf [E, H, I/32]; activations MXFP8 (W4A8)
    "nvfp4": w13 packed E2M1 [E, 2I, H/2] + w13_sf uint8 E4M3 [E, 2I, H/16]
             + w13_gs float32 [E]; w2 [E, H, I/2] + w2_sf [E, H, I/16]
             + w2_gs [E]; activations NVFP4 (per-token global scale at L1,
             ``l2_activation_scale`` at L2)
"""

import numpy as np

from . import codecs, quant
from .dispatch import slot_experts

FORMATS = ("bf16", "mxfp8", "mxfp4", "nvfp4")

_E4M3_LUT = codecs.e4m3_decode(np.arange(256, dtype=np.uint8))
_E2M1_LUT = codecs.e2m1_decode(np.arange(16, dtype=np.uint8))


def sigmoid(z):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def activation(g, u, clamp=None, alpha=1.0, beta=0.0):
    """``MegaMoEActivation`` swiglu, float64."""
    if clamp is not None:
        g = np.minimum(g, clamp)
        u = np.clip(u, -clamp, clamp)
    return g * sigmoid(alpha * g) * (u + beta)


# --------------------------------------------------------------------------
# dequantisation of one expert's canonical weights
# --------------------------------------------------------------------------

def _deq_mx(codes, sf, elem):
    vals = _E4M3_LUT[codes] if elem == "e4m3" else _E2M1_LUT[codecs.fp4_unpack(codes)]
    K = vals.shape[-1]
    s = codecs.ue8m0_decode(sf)
    return (vals.reshape(vals.shape[:-1] + (K // 32, 32)) * s[..., None]).reshape(vals.shape)


def _deq_nv(codes, sf, gs):
    vals = _E2M1_LUT[codecs.fp4_unpack(codes)]
    K = vals.shape[-1]
    s = _E4M3_LUT[sf]
    out = (vals.reshape(vals.shape[:-1] + (K // 16, 16)) * s[..., None]).reshape(vals.shape)
    return out * np.float64(gs)


def dequant_weight(fmt, w, name, e):
    """float64 [N, K] of expert ``e``'s ``name`` ("w13" or "w2")."""
    if fmt == "bf16":
        return codecs.bf16_decode(w[name][e])
    if fmt == "mxfp8":
        return _deq_mx(w[name][e], w[name + "_sf"][e], "e4m3")
    if fmt == "mxfp4":
        return _deq_mx(w[name][e], w[name + "_sf"][e], "e2m1")
    if fmt == "nvfp4":
        return _deq_nv(w[name][e], w[name + "_sf"][e], w[name + "_gs"][e])
    raise ValueError(fmt)


# --------------------------------------------------------------------------
# activation quantisers (dispatch side and L2 input)
# --------------------------------------------------------------------------

def quantize_x(fmt, x_bits):
    """Dispatch quantisation of BF16 rows -> float64 values the L1 GEMM sees."""
    x32 = codecs.bf16_decode(x_bits).astype(np.float32)
    if fmt == "bf16":
        return x32.astype(np.float64)
    if fmt in ("mxfp8", "mxfp4"):
        q, c = quant.mx_quantize(x32, "e4m3")
        return quant.mx_dequantize(q, c, "e4m3")
    if fmt == "nvfp4":
        g = quant.nvfp4_global_scale(np.abs(x32).max(axis=-1))
        q, bs = quant.nvfp4_quantize(x32, g)
        return quant.nvfp4_dequantize(q, bs, g)
    raise ValueError(fmt)


def quantize_l2_input(fmt, a, l2_activation_scale=1.0):
    """L2-input quantisation of float64 activations (taken through float32)."""
    a32 = np.asarray(a, dtype=np.float64).astype(np.float32)
    if fmt == "bf16":
        return codecs.bf16_decode(codecs.bf16_encode_f32(a32))
    if fmt in ("mxfp8", "mxfp4"):
        q, c = quant.mx_quantize(a32, "e4m3")
        return quant.mx_dequantize(q, c, "e4m3")
    if fmt == "nvfp4":
        g = np.full(a32.shape[:-1], np.float32(l2_activation_scale), dtype=np.float32)
        q, bs = quant.nvfp4_quantize(a32, g)
        return quant.nvfp4_dequantize(q, bs, g)
    raise ValueError(fmt)


# --------------------------------------------------------------------------
# the layer
# --------------------------------------------------------------------------

def post_expert_norm(y, gamma, eps):
    """The Muse-Spark MegaMoE page's post-expert RMSNorm, which its kernel
    applies to the layer output (``post_expert_norm_gamma``,
    ``post_expert_norm_eps``; the caller folds a zero-centred gain into
    gamma): y / sqrt(mean over H of y^2 + eps) * gamma, float64."""
    y = np.asarray(y, dtype=np.float64)
    return y / np.sqrt(np.mean(y * y, axis=-1, keepdims=True) + eps) * np.asarray(gamma, dtype=np.float64)


def weight_on_input(x_bits, topk_weights):
    """``apply_router_weight_on_input`` ("fused_moe" page, FusedMoE): each
    token's (single) routing weight multiplies its BF16 input row, in float32
    with one round to BF16, before the experts; the combine then weighs the
    slot by 1."""
    x32 = codecs.bf16_decode(x_bits).astype(np.float32)
    w32 = np.asarray(topk_weights, dtype=np.float32)[:, :1]
    return codecs.bf16_encode_f32((x32 * w32).astype(np.float32))


def moe_reference(fmt, x_bits, topk_ids, topk_weights, w, *, num_shared=0,
                  expert_start=0, num_local=None, act=None,
                  l2_activation_scale=1.0, tokens=None, norm=None, router_weight_on_input=False):
    """float64 output [len(tokens), H] (all tokens if ``tokens`` is None).

    ``act`` is a dict with keys clamp (None or float), alpha, beta.
    ``l2_activation_scale`` is the NVFP4 L2 global input scale.  ``norm``:
    None or (gamma [H], eps), the post-expert RMSNorm of the output.
    ``router_weight_on_input``: top_k = 1 and no shared expert; the routing
    weight scales the input instead of the expert output.
    """
    if router_weight_on_input:
        if np.asarray(topk_ids).shape[1] != 1 or num_shared:
            raise ValueError("router weight on the input needs top_k = 1 and no shared expert")
        x_bits = weight_on_input(x_bits, topk_weights)
        topk_weights = np.ones_like(np.asarray(topk_weights, dtype=np.float64))
        y = moe_reference(fmt, x_bits, topk_ids, topk_weights, w, num_shared=0, expert_start=expert_start,
                          num_local=num_local, act=act, l2_activation_scale=l2_activation_scale,
                          tokens=tokens)
        return y if norm is None else post_expert_norm(y, *norm)
    if fmt not in FORMATS:
        raise ValueError(fmt)
    act = dict(act or {})
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, H = x_bits.shape
    E_all = w["w13"].shape[0]
    if num_local is None:
        num_local = E_all - num_shared
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    xs = quantize_x(fmt, x_bits[tok])                          # [n, H]
    exp = slot_experts(np.asarray(topk_ids)[tok], num_shared, expert_start, num_local)
    k = np.asarray(topk_ids).shape[1]
    wts = np.concatenate(
        [np.asarray(topk_weights, dtype=np.float64)[tok],
         np.ones((tok.size, num_shared))], axis=1)
    y = np.zeros((tok.size, H), dtype=np.float64)
    for e in np.unique(exp[exp >= 0]):
        r, j = np.nonzero(exp == e)
        W13 = dequant_weight(fmt, w, "w13", e)                 # [2I, H]
        I = W13.shape[0] // 2
        h = xs[r] @ W13.T                                      # [n, 2I]
        del W13
        a = activation(h[:, :I], h[:, I:], act.get("clamp"),
                       act.get("alpha", 1.0), act.get("beta", 0.0))
        a_hat = quantize_l2_input(fmt, a, l2_activation_scale)
        W2 = dequant_weight(fmt, w, "w2", e)                   # [H, I]
        o = a_hat @ W2.T                                       # [n, H]
        np.add.at(y, r, wts[r, j][:, None] * o)
    return y if norm is None else post_expert_norm(y, *norm)


def slot_activations(fmt, x_bits, topk_ids, w, *, num_shared=0, expert_start=0, num_local=None, act=None,
                     tokens=None):
    """The values the L2-input quantiser receives: for every slot that
    reaches a local expert, a = act(g, u) with [g; u] = Deq(W13_e) @ x_hat,
    float64 (the steps of ``moe_reference`` up to the L2-input
    quantisation).

    Returns (slots, experts, a): flat slot ids t * k' + j (t the token's
    index in ``x_bits``) [n], their local experts [n] and the activations
    [n, I], ordered by expert, then by slot.  ``tokens``: restrict to these
    token indices."""
    act = dict(act or {})
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T = x_bits.shape[0]
    E_all = w["w13"].shape[0]
    if num_local is None:
        num_local = E_all - num_shared
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    xs = quantize_x(fmt, x_bits[tok])
    exp = slot_experts(np.asarray(topk_ids)[tok], num_shared, expert_start, num_local)
    kk = exp.shape[1]
    slots, experts, acts = [], [], []
    for e in np.unique(exp[exp >= 0]):
        r, j = np.nonzero(exp == e)
        W13 = dequant_weight(fmt, w, "w13", e)
        I = W13.shape[0] // 2
        h = xs[r] @ W13.T
        acts.append(activation(h[:, :I], h[:, I:], act.get("clamp"), act.get("alpha", 1.0), act.get("beta", 0.0)))
        slots.append(tok[r] * kk + j)
        experts.append(np.full(r.size, e))
    if not slots:
        I = w["w2"].shape[-1] * (2 if fmt in ("mxfp4", "nvfp4") else 1)
        return np.zeros(0, np.int64), np.zeros(0, np.int64), np.zeros((0, I))
    return np.concatenate(slots), np.concatenate(experts), np.concatenate(acts)
