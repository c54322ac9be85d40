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


class WorkspaceReader:
    """The intermediate buffers of the last forward of ``layer`` with ``T``
    tokens (and the BLOCK_M it ran with), read back through
    moe_workspace_layout."""

    def __init__(self, layer, T, block_m=0):
        self.layer, self.T = layer, T
        self.fmt, self.I, self.H = layer.fmt, layer.inter, layer.hidden
        self.E = layer.num_experts
        self.kk = layer.top_k + layer.num_shared
        self.S = T * self.kk
        self.lay = moe._lib.moe_workspace_layout(layer.fmt, T, layer.hidden, layer.inter, layer.top_k,
                                                 layer.num_local_experts, layer.num_shared, block_m,
                                                 layer.workspace.numel())
        self.bm = self.lay["block_m"]
        self.ws = layer.workspace.cpu().numpy()

    def bytes(self, name, n, offset=0):
        o = self.lay[name]
        assert o >= 0, name
        return self.ws[o + offset:o + offset + n]

    def i32(self, name, n):
        return self.bytes(name, 4 * n).view(np.int32)

    def dispatch(self):
        offsets = self.i32("offsets", self.E + 1)
        M = int(offsets[-1])
        return {"counts": self.i32("counts", self.E), "offsets": offsets,
                "sorted_slot": self.i32("sorted_slot", M), "slot_row": self.i32("slot_row", self.S),
                "tile_expert": self.i32("tile_expert", M // self.bm)}

    def xq(self):
        """dispatch-quantised x: (codes [T, H] unpacked, scales [T, H/grp],
        token scales [T] or None)"""
        T, H = self.T, self.H
        if self.fmt == "nvfp4":
            packed = self.bytes("xq", T * H // 2).reshape(T, H // 2)
            codes = np.stack([packed & 0xF, packed >> 4], -1).reshape(T, H)
            return codes, self.bytes("xq_sf", T * H // 16).reshape(T, H // 16), \
                self.bytes("x_tok", 4 * T).view(np.float32)
        return self.bytes("xq", T * H).reshape(T, H), self.bytes("xq_sf", T * H // 32).reshape(T, H // 32), None

    def a1_planes(self, rows):
        """x's block scales of sorted rows [0, rows), [rows, H/grp]"""
        grp = 16 if self.fmt == "nvfp4" else 32
        p = self.lay["sf_plane"]
        return np.stack([self.bytes("a1_sf", rows, b * p) for b in range(self.H // grp)], 1)

    def l2_input(self, rows):
        """The L2 input of sorted rows ``rows``: (codes [n, I] unpacked, or
        BF16 bits; scales [n, I/grp] or None)"""
        rows = np.asarray(rows, dtype=np.int64)
        I, ld = self.I, self.lay["a2_ld"]
        if self.fmt == "bf16":
            bm = self.bm
            base = self.lay["a2"]
            full = self.ws[base:base + (int(rows.max()) // bm + 1) * bm * I * 2].view(np.uint16)
            full = full.reshape(-1, I // 32, bm, 32).transpose(0, 2, 1, 3).reshape(-1, I)
            return full[rows], None
        a2 = self.ws[self.lay["a2"]:self.lay["a2"] + (int(rows.max()) + 1) * ld].reshape(-1, ld)[rows]
        grp = 16 if self.fmt == "nvfp4" else 32
        p, b0 = self.lay["sf_plane"], self.lay["a2_sf"]
        sf = np.stack([self.ws[b0 + b * p + rows] for b in range(I // grp)], 1)
        if self.fmt == "nvfp4":
            a2 = np.stack([a2 & 0xF, a2 >> 4], -1).reshape(len(rows), I)
        return a2, sf
