"""Helpers of the GPU tests: upload canonical arrays, run the HIP layer through
the C ABI, bring results back as NumPy."""

import numpy as np
import torch

import expert_gemms_amd as moe


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def x_dev(x_bits):
    return dev(x_bits).view(torch.bfloat16)


def run_layer(fmt, x_bits, ids, wts, w, *, num_shared=0, expert_start=0, num_local=None, block_m=0,
              act=None, w2_input_scale=None, max_tokens=None, norm=None, weight_on_input=False):
    """Canonical NumPy inputs -> float64 NumPy output of moe_forward."""
    T, H = x_bits.shape
    E_all = w["w13"].shape[0]
    num_local = E_all - num_shared if num_local is None else num_local
    I = w["w2"].shape[2] * (2 if fmt in ("mxfp4", "nvfp4") else 1)
    layer = moe.FusedMoE(fmt, H, I, num_local, ids.shape[1], num_shared=num_shared,
                         expert_start=expert_start, max_tokens=max(T, max_tokens or 0, 1), act=act)
    layer.load_canonical(dev(w["w13"]), dev(w["w2"]),
                         dev(w["w13_sf"]) if "w13_sf" in w else None,
                         dev(w["w2_sf"]) if "w2_sf" in w else None,
                         dev(w["w13_gs"]) if "w13_gs" in w else None,
                         dev(w["w2_gs"]) if "w2_gs" in w else None,
                         w2_input_scale=None if w2_input_scale is None else torch.from_numpy(w2_input_scale))
    gamma = None if norm is None else torch.from_numpy(np.asarray(norm[0], dtype=np.float32)).cuda()
    out = layer.forward(x_dev(x_bits), dev(ids.astype(np.int32)), dev(wts.astype(np.float32)), block_m=block_m,
                        norm_gamma=gamma, norm_eps=0.0 if norm is None else float(norm[1]),
                        weight_on_input=weight_on_input)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), layer
