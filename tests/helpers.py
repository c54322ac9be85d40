"""Test-side helpers: canonical weight sets built with the oracle's quantisers
from the seeded float32 sources, and the comparison bar of the layer output.

Weights handed to both the HIP path and the oracle come from here, so no
oracle input is ever produced by the HIP path.
"""

import numpy as np
import torch

from oracle import codecs, quant
from synth import gen_weight_f32, bf16_bits


def quantize_weight(fmt, w32):
    """float32 [N, K] -> dict of canonical arrays for one expert."""
    if fmt == "bf16":
        return {"w": bf16_bits(torch.from_numpy(np.ascontiguousarray(w32)).to(torch.bfloat16))}
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
