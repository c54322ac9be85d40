"""Test-side helpers: canonical weight sets built with the oracle's quantisers
from the seeded float32 sources, and the comparison bar of the layer output.

Weights handed to both the HIP path and the oracle come from here, so no
oracle input is ever produced by the HIP path.
"""

import numpy as np
import torch

import itertools

from oracle import codecs, quant
from oracle.dispatch import slot_experts
from oracle.moe import activation, dequant_weight, quantize_x
from synth import gen_weight_f32, bf16_bits


def quantize_weight(fmt, w32):
    """float32 [N, K] -> dict of canonical arrays for one expert (the
    oracle's codecs and quantisers only: NumPy, safe in forked workers)."""
    if fmt == "bf16":
        return {"w": codecs.bf16_encode_f32(np.ascontiguousarray(w32, dtype=np.float32))}
    if fmt == "mxfp8":
        q, c = quant.mx_quantize(w32, "e4m3")
        return {"w": q, "sf": c}
    if fmt == "mxfp4":
        q, c = quant.mx_quantize(w32, "e2m1")
        return {"w": codecs.fp4_pack(q), "sf": c}
    if fmt == "nvfp4":
        g = quant.nvfp4_global_scale(np.array(np.abs(w32).max(), dtype=np.float32))
        q, bs = quant.nvfp4_quantize(w32, np.full(w32.shape[0], g, dtype=np.float32))
        return {"w": codecs.fp4_pack(q), "sf": bs, "gs": np.float32(g)}
    raise ValueError(fmt)


def make_weights(cfg, fmt=None, seed=0, sources=None):
    """Canonical weight dict for all E + num_shared experts of ``cfg``:
    keys w13, w2 (+ w13_sf, w2_sf, + w13_gs, w2_gs for NVFP4)."""
    fmt = fmt or cfg.fmt
    E = cfg.E + cfg.num_shared
    out = {}
    for name in ("w13", "w2"):
        parts = []
        for e in range(E):
            src = sources[name][e] if sources is not None else gen_weight_f32(cfg, name, e, seed)
            parts.append(quantize_weight(fmt, src))
        out[name] = np.stack([p["w"] for p in parts])
        if "sf" in parts[0]:
            out[name + "_sf"] = np.stack([p["sf"] for p in parts])
        if "gs" in parts[0]:
            out[name + "_gs"] = np.array([p["gs"] for p in parts], dtype=np.float32)
    return out


# Parity figures of this session (GPU tests), printed one line per case at
# the end of the run by tests/conftest.py.
PARITY = []


def record_parity(case, **stats):
    PARITY.append((case, stats))


def rescue_cap(n_tokens):
    """Tokens the boundary-decision rule may accept in one comparison: half a
    percent of them, and at least one."""
    return max(1, int(0.005 * n_tokens))


def bf16_half_ulp(y):
    """Half a unit in the last place of BF16 at |y| (the output container's
    own rounding)."""
    a = np.abs(np.asarray(y, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 2.0 ** -126)))
    return np.exp2(np.maximum(e, -126) - 8)


TOL = {"bf16": 1e-2, "mxfp8": 3e-2, "mxfp4": 3e-2, "nvfp4": 3e-2}


def check_output(fmt, y_gpu, y_ref, rms=None):
    """The layer's output bar: |y_gpu - y_ref| <= tol * RMS(y_ref) + half a
    BF16 ulp of y_ref, with tol 1e-2 (BF16) or 3e-2 (MX, NVFP4).  The BF16
    output container alone rounds by up to half an ulp, which for the largest
    outputs exceeds 1e-2 * RMS; the bar charges the computation with
    everything beyond that rounding.  Returns (max err / RMS, worst excess)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if rms is None else rms
    err = np.abs(y_gpu - y_ref)
    bound = TOL[fmt] * rms + bf16_half_ulp(y_ref)
    excess = float((err - bound).max()) if err.size else 0.0
    return float(err.max() / rms) if err.size and rms > 0 else 0.0, excess


def error_summary(y_gpu, y_ref):
    """The output error apart from the BF16 container's own rounding:
    max(|y_gpu - y_ref| - half an ulp of y_ref) / RMS (the computation's
    share, <= 0 when every output is within its own rounding), and the
    largest distance from the round-to-nearest-even BF16 of the oracle, in
    BF16 ulps of that value."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if not y_ref.size:
        return {"excess_over_rounding_per_rms": 0.0, "max_ulps_from_rne": 0.0}
    rms = float(np.sqrt(np.mean(y_ref ** 2))) or 1.0
    rne = codecs.bf16_round_f64(y_ref)
    ulp = 2.0 * bf16_half_ulp(rne)
    return {"excess_over_rounding_per_rms": float((np.abs(y_gpu - y_ref) - bf16_half_ulp(y_ref)).max() / rms),
            "max_ulps_from_rne": float((np.abs(y_gpu - rne) / ulp).max())}


# --------------------------------------------------------------------------
# L2-input quantisation decisions that sit on a boundary
# --------------------------------------------------------------------------
# The L2 input is quantised from the activations: its block scales and
# element codes are integers decided by floating point.  Both sides decide in
# float32 (the method's precision), but from activations summed in different
# orders and precisions (the GPU's MFMAs vs float64), so a value lying closer
# to a decision boundary (an element's rounding midpoint, the amax where a
# block scale changes) than the GPU's evaluation error has two valid
# quantisations.  One flipped element moves its contribution by a whole code
# step, which for a token with few L2 terms can exceed the bar.  For tokens
# over the bar, the check recomputes that token with the other valid choice
# of each such decision (every combination) and accepts it if one meets the
# bar; every other token is compared as computed.  The evaluation error bound
# per activation (_act_error_rows): the float32 accumulation bound of g and u
# (accumulation_bound), for the MX formats plus the scaled MFMA's own
# (MX_MFMA_STEP_BOUND), carried through the activation, plus 2^-18 relative
# (hardware exp and reciprocal).

def accumulation_bound(fmt, K):
    """Bound, relative to the sum of |products|, on the float32 rounding
    error of one L1 output (K products): the GPU adds one MFMA K-step's
    products (16 for BF16 and NVFP4, 64 for the scaled MX MFMA) into a
    float32 accumulator at a time, at most one rounding (2^-24 relative) per
    step, plus the K-split parts and NVFP4's two scale products; doubled for
    margin."""
    kstep = 64 if fmt in ("mxfp8", "mxfp4") else 16
    return 2.0 * (K // kstep + 4) * 2.0 ** -24


# The scaled MFMA (v_mfma_scale_f32_32x32x64_f8f6f4, the MX formats' L1 and
# L2) does not add its 64 products at float32 precision: measured with an
# in-bounds probe on MI355X, one instruction's result is exact while its
# products span a few binades, and otherwise off by at most 2^-11.06 times
# the power of two at or below its largest |product| (one instruction, codes
# drawn over the whole E4M3 range; 2^-12.7 for normal-like data), FP8 x FP8
# and FP8 x FP4 alike.  The bound taken per 64-wide K-step is 2^-10 times
# the step's largest |product| (twice the worst measurement).  The BF16 and
# FP16 MFMAs (BF16 and NVFP4 layers) keep the float32 bound above.
MX_MFMA_STEP_BOUND = 2.0 ** -10


def step_max_products(X, W, step=64):
    """[n, N]: for every output (row of X, row of W), the sum over its
    64-wide K-steps of the step's largest |product|."""
    n, K = X.shape
    N = W.shape[0]
    st = K // step
    Wa = np.abs(W).reshape(N, st, step)
    out = np.zeros((n, N))
    for i in range(n):
        out[i] = (Wa * np.abs(X[i]).reshape(st, step)[None]).max(-1).sum(-1)
    return out


def _act_error_rows(fmt, W13, X, act, exact=False):
    """float64 activations a [n, I] of n slots of one expert (inputs X [n, H])
    and a bound on the error with which the GPU evaluates them: the bound
    on g and u (float32 accumulation; for the MX formats plus the scaled
    MFMA's per-step bound; with ``exact``, inputs whose L1 sums every path
    computes exactly, only NVFP4's two float32 scale products and float64
    noise) carried
    through the activation, plus 2^-18 relative for the hardware exp and
    reciprocal."""
    I = W13.shape[0] // 2
    h = X @ W13.T
    if exact:
        # NVFP4's float32 scale products, and the oracle's own float64
        # evaluation noise (an exactly zero sum can come out of the float64
        # matmul as +-1e-17, on either side of zero)
        eh = np.abs(h) * (4.0 * 2.0 ** -24 if fmt == "nvfp4" else 0.0) + \
            (np.abs(X) @ np.abs(W13).T) * 2.0 ** -40
    else:
        eh = (np.abs(X) @ np.abs(W13).T) * accumulation_bound(fmt, W13.shape[1])
        if fmt in ("mxfp8", "mxfp4"):
            eh = eh + MX_MFMA_STEP_BOUND * step_max_products(X, W13)
    f = lambda g, u: activation(g, u, act.get("clamp"), act.get("alpha", 1.0), act.get("beta", 0.0))
    g, u, eg, eu = h[:, :I], h[:, I:], eh[:, :I], eh[:, I:]
    a = f(g, u)
    da = np.max([np.abs(f(g + sg * eg, u + su * eu) - a) for sg in (-1, 1) for su in (-1, 1)], axis=0)
    return a, da + np.ldexp(np.abs(a), -18)


def _act_error(W13, xs, act, fmt="mxfp8"):
    """_act_error_rows for one slot."""
    a, da = _act_error_rows(fmt, W13, xs[None, :], act)
    return a[0], da[0]


def slot_l2_inputs(fmt, x_bits, ids, w, *, num_shared=0, expert_start=0, num_local=None, act=None, tokens=None,
                   exact=False):
    """(slots, experts, a, da): the oracle's activations of every live slot
    (oracle.moe.slot_activations) and a bound on the error with which the
    GPU computes them (_act_error_rows; ``exact`` for inputs whose L1 sums
    are exact on the GPU)."""
    from oracle.moe import slot_activations
    act = dict(act or {})
    slots, experts, a = slot_activations(fmt, x_bits, ids, w, num_shared=num_shared, expert_start=expert_start,
                                         num_local=num_local, act=act, tokens=tokens)
    kk = np.asarray(ids).shape[1] + num_shared
    da = np.zeros_like(a)
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        X = quantize_x(fmt, np.asarray(x_bits)[slots[sel] // kk])
        _, da[sel] = _act_error_rows(fmt, dequant_weight(fmt, w, "w13", e), X, act, exact=exact)
    return slots, experts, a, da


def _allowed(dec, enc, v, dv, got):
    """Element codes ``got`` that some value in [v - dv, v + dv] encodes to:
    the decoded value lies between those of the interval's ends (encoding
    is monotone), and a zero's sign bit is one of the interval's signs."""
    lo, hi = enc(v - dv), enc(v + dv)
    gv, lv, hv = dec(got), dec(lo), dec(hi)
    ok = (gv >= np.minimum(lv, hv)) & (gv <= np.maximum(lv, hv))
    sign_bit = 0x8000 if got.dtype == np.uint16 else (0x8 if dec is codecs.e2m1_decode else 0x80)
    neg = (got & sign_bit) != 0
    zero = gv == 0
    ok &= ~zero | np.where(neg, v - dv <= 0, v + dv >= 0)
    return ok


def l2_code_check(fmt, codes, scales, a, da, g2=1.0):
    """The GPU's L2-input codes of n slots (``codes`` [n, I]: BF16 bits, or
    unpacked E4M3 / E2M1 codes; ``scales`` [n, I/32] UE8M0 or [n, I/16]
    E4M3) against the oracle's quantiser applied to the oracle's float32
    activations ``a`` (evaluation error bound ``da``).  A code or block scale
    may differ from the oracle's only where the activation lies within its
    error bound of a decision boundary, i.e. where some value within the
    bound is quantised to the GPU's decision.  Returns counts: elements,
    element flips (values unlike the oracle's, all of them boundary cases),
    zero-sign flips (+0 against -0 where the value is within its bound of
    zero), blocks, scale flips, and ``unexplained`` (differences not so
    covered; must be 0)."""
    a = np.asarray(a, dtype=np.float64)
    da = np.asarray(da, dtype=np.float64)
    n, I = a.shape
    a32 = a.astype(np.float32)
    if fmt == "bf16":
        own = codecs.bf16_encode_f32(a32)
        f32 = lambda v: codecs.bf16_encode_f32(np.asarray(v).astype(np.float32))
        ok = _allowed(codecs.bf16_decode, f32, a, da, codes)
        vdiff = codecs.bf16_decode(codes) != codecs.bf16_decode(own)
        return {"elements": int(a.size), "element_flips": int(vdiff.sum()),
                "zero_sign_flips": int(((codes != own) & ~vdiff).sum()), "blocks": 0,
                "scale_flips": 0, "unexplained": int((~ok).sum())}
    grp = 16 if fmt == "nvfp4" else 32
    nb = I // grp
    blk = a.reshape(n, nb, grp)
    dblk = da.reshape(n, nb, grp)
    got_c = np.asarray(codes).reshape(n, nb, grp)
    got_s = np.asarray(scales).reshape(n, nb)
    amax_lo = np.maximum(np.abs(blk) - dblk, 0.0).max(-1)
    amax_hi = (np.abs(blk) + dblk).max(-1)
    if fmt in ("mxfp8", "mxfp4"):
        own_q, own_s = quant.mx_quantize(a32, "e4m3")
        s_lo = quant.mx_scale_codes(amax_lo.astype(np.float32), "e4m3")
        s_hi = quant.mx_scale_codes(amax_hi.astype(np.float32), "e4m3")
        scale_ok = (got_s >= s_lo) & (got_s <= s_hi)
        # elements under the GPU's own block scale
        mul = np.where(got_s > 0, np.ldexp(1.0, 127 - got_s.astype(np.int64)), 0.0)[..., None]
        ok = _allowed(codecs.e4m3_decode, codecs.e4m3_encode, blk * mul, dblk * mul, got_c)
        ok |= (got_s == 0)[..., None] & (got_c == 0)
    else:
        g = np.float32(g2)
        own_q, own_s = quant.nvfp4_quantize(a32, np.full(n, g, dtype=np.float32))
        six_g = np.float32(np.float32(6.0) * g)
        s_lo = codecs.e4m3_encode((amax_lo / float(six_g)).astype(np.float32))
        s_hi = codecs.e4m3_encode((amax_hi / float(six_g)).astype(np.float32))
        sv = codecs.e4m3_decode(got_s)
        scale_ok = (sv >= codecs.e4m3_decode(s_lo)) & (sv <= codecs.e4m3_decode(s_hi)) & (got_s < 0x80)
        r = np.where(sv > 0, (np.float32(1.0) / np.maximum(sv * g, 1e-30).astype(np.float32)).astype(np.float64),
                     0.0)[..., None]
        ok = _allowed(codecs.e2m1_decode, codecs.e2m1_encode, blk * r, dblk * r, got_c)
        ok |= (sv == 0)[..., None] & ((got_c & 0x7) == 0)
    own_q = own_q.reshape(n, nb, grp)
    same_scale = got_s == own_s
    dec = codecs.e4m3_decode if fmt in ("mxfp8", "mxfp4") else codecs.e2m1_decode
    vdiff = dec(got_c) != dec(own_q)
    return {"elements": int(a.size), "element_flips": int((vdiff & same_scale[..., None]).sum()),
            "zero_sign_flips": int(((got_c != own_q) & ~vdiff & same_scale[..., None]).sum()),
            "blocks": int(got_s.size), "scale_flips": int((~same_scale).sum()),
            "unexplained": int((~ok).sum() + (~scale_ok).sum())}


def decision_alternatives(fmt, a, da, g2=1.0):
    """[(offset, change of the dequantised L2 input block)] for the
    boundary decisions of one slot's L2 input (float64 activations ``a`` [I]
    with evaluation error bound ``da``)."""
    a32 = np.asarray(a, dtype=np.float64).astype(np.float32)
    out = []
    if fmt in ("mxfp8", "mxfp4"):
        G = 32
        for off in range(0, a32.size, G):
            v = a32[off:off + G].astype(np.float64)
            d = da[off:off + G]
            i = int(np.abs(v).argmax())
            amax = abs(v[i])
            if amax == 0.0:
                continue
            q, c = quant.mx_quantize(v, "e4m3")
            own = quant.mx_dequantize(q, c, "e4m3")
            lo = int(quant.mx_scale_codes(amax - d[i], "e4m3"))
            hi = int(quant.mx_scale_codes(amax + d[i], "e4m3"))
            if lo != hi:                       # the block scale itself
                other = hi if int(c[0]) == lo else lo
                q2, c2 = quant.mx_quantize(v, "e4m3", codes=[other])
                out.append((off, quant.mx_dequantize(q2, c2, "e4m3") - own))
                continue
            s = np.ldexp(1.0, 127 - int(c[0]))
            sv, ds = v * s, d * s
            qlo, qhi = codecs.e4m3_encode(sv - ds), codecs.e4m3_encode(sv + ds)
            for k in np.nonzero(qlo != qhi)[0]:  # element rounding
                other = qhi[k] if q[k] == qlo[k] else qlo[k]
                delta = np.zeros(G)
                delta[k] = (codecs.e4m3_decode(np.uint8(other)) - codecs.e4m3_decode(q[k])) / s
                out.append((off, delta))
    elif fmt == "nvfp4":
        G = 16
        g = np.float32(g2)
        six_g = np.float32(np.float32(6.0) * g)
        for off in range(0, a32.size, G):
            v = a32[off:off + G]
            d = da[off:off + G]
            i = int(np.abs(v).argmax())
            amax = float(abs(v[i]))
            if amax == 0.0:
                continue
            q, bs = quant.nvfp4_quantize(v, g)
            own = quant.nvfp4_dequantize(q, bs, g)
            t, dt = amax / float(six_g), d[i] / float(six_g)
            lo = int(codecs.e4m3_encode(np.float32(t - dt)))
            hi = int(codecs.e4m3_encode(np.float32(t + dt)))
            if lo != hi:
                other = hi if int(bs[0]) == lo else lo
                q2, bs2 = quant.nvfp4_quantize(v, g, bs=[other])
                out.append((off, quant.nvfp4_dequantize(q2, bs2, g) - own))
                continue
            bsv = float(codecs.e4m3_decode(bs[0]))
            if bsv == 0.0:
                continue
            r = 1.0 / (bsv * float(g))
            pv, dp = v.astype(np.float64) * r, d * r
            qlo, qhi = codecs.e2m1_encode(pv - dp), codecs.e2m1_encode(pv + dp)
            for k in np.nonzero(qlo != qhi)[0]:
                other = qhi[k] if q[k] == qlo[k] else qlo[k]
                delta = np.zeros(G)
                delta[k] = (codecs.e2m1_decode(np.uint8(other)) - codecs.e2m1_decode(q[k])) * bsv * float(g)
                out.append((off, delta))
    return out


def check_layer(fmt, y_gpu, y_ref, x_bits, ids, wts, w, *, num_shared=0, expert_start=0, num_local=None,
                act=None, g2=1.0, tokens=None, max_decisions=12, norm=None, y_pre=None, name=None):
    """check_output, plus the boundary-decision rule above for tokens over
    the bar (every combination of a token's boundary decisions when there are
    at most ``max_decisions``, else a greedy search).  ``tokens``: the token
    index of each row (default: all rows in order).  Returns (max err / RMS as computed, worst excess after the rule,
    number of tokens accepted under another valid decision)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(y_ref ** 2)))
    rel, excess = check_output(fmt, y_gpu, y_ref, rms=rms)

    def done(worst, rescued):
        if name is not None:
            record_parity(name, tokens=int(y_ref.shape[0]), max_err_per_rms=rel, worst_excess=worst,
                          rescued=rescued, rescue_cap=rescue_cap(y_ref.shape[0]), **error_summary(y_gpu, y_ref))
        return rel, worst, rescued

    if excess <= 0 or fmt == "bf16":
        return done(excess, 0)

    def row_excess(yg, yr):
        return float((np.abs(yg - yr) - (TOL[fmt] * rms + bf16_half_ulp(yr))).max())

    def post(r, delta):
        """the oracle row r with the pre-norm change delta"""
        if norm is None:
            return y_ref[r] + delta
        from oracle.moe import post_expert_norm
        return post_expert_norm(y_pre[r] + delta, *norm)

    tok = np.arange(y_ref.shape[0]) if tokens is None else np.asarray(tokens)
    E_all = w["w13"].shape[0]
    num_local = E_all - num_shared if num_local is None else num_local
    ids = np.asarray(ids)
    k = ids.shape[1]
    act = dict(act or {})
    cache = {}
    worst, rescued = -np.inf, 0
    for r in range(y_ref.shape[0]):
        ex = row_excess(y_gpu[r], y_ref[r])
        if ex <= 0:
            worst = max(worst, ex)
            continue
        t = int(tok[r])
        exp = slot_experts(ids[t:t + 1], num_shared, expert_start, num_local)[0]
        xs = quantize_x(fmt, np.asarray(x_bits)[t:t + 1])[0]
        deltas = []
        for j, e in enumerate(exp):
            if e < 0:
                continue
            if e not in cache:
                cache[e] = (dequant_weight(fmt, w, "w13", e), dequant_weight(fmt, w, "w2", e))
            W13, W2 = cache[e]
            a, da = _act_error(W13, xs, act, fmt)
            wj = float(wts[t, j]) if j < k else 1.0
            for off, dv in decision_alternatives(fmt, a, da, g2):
                deltas.append(wj * (W2[:, off:off + dv.size] @ dv))
        best = ex
        if 0 < len(deltas) <= max_decisions:
            # every combination
            for n in range(1, len(deltas) + 1):
                for combo in itertools.combinations(deltas, n):
                    best = min(best, row_excess(y_gpu[r], post(r, np.sum(combo, axis=0))))
        elif deltas:
            # too many to enumerate: add, one at a time, the decision that
            # brings the oracle closest (2-norm) to the GPU row, while it helps
            acc = np.zeros_like(y_ref[r])
            left = list(range(len(deltas)))
            for _ in range(max_decisions):
                cur = post(r, acc)
                if row_excess(y_gpu[r], cur) <= 0 or not left:
                    break
                norms = [np.linalg.norm(y_gpu[r] - post(r, acc + deltas[i])) for i in left]
                i = int(np.argmin(norms))
                if norms[i] >= np.linalg.norm(y_gpu[r] - cur):
                    break
                acc = acc + deltas[left.pop(i)]
            best = min(best, row_excess(y_gpu[r], post(r, acc)))
        if best <= 0:
            rescued += 1
        worst = max(worst, best)
    return done(worst, rescued)
