"""``FusedMoE``: kernel-layout weights plus a workspace for ``moe_forward``.

The holder mirrors DeepGemmMegaMoEExperts on the DeepGEMM MegaMoE experts
page (weights kept in the kernel layout, a buffer sized for a maximum token
count, ``forward(hidden_states, topk_weights, topk_ids)``), with the
allocations made by torch and the computation done by the library.
"""

import torch

from . import _lib


def _elem_bytes(fmt):
    return {"bf16": 2.0, "mxfp8": 1.0, "mxfp4": 0.5, "nvfp4": 0.5}[fmt]


class FusedMoE:
    def __init__(self, fmt, hidden, inter, num_local_experts, top_k, *, num_shared=0, expert_start=0,
                 max_tokens, act=None, device=None):
        self.fmt = fmt
        self.hidden, self.inter = hidden, inter
        self.num_local_experts, self.num_shared = num_local_experts, num_shared
        self.top_k, self.expert_start = top_k, expert_start
        self.max_tokens = max_tokens
        self.act = act
        self.device = torch.device(device or "cuda")
        self.num_experts = num_local_experts + num_shared
        nbytes = _lib.moe_workspace_bytes(fmt, max_tokens, hidden, inter, num_local_experts,
                                          num_shared, top_k, 0)
        if nbytes == 0:
            raise ValueError("invalid layer shape")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.w13_k = self.w2_k = self.w13_sf_k = self.w2_sf_k = None
        self.w13_gs = self.w2_gs = None
        self.l2_activation_scale = 1.0
        self.norm_gamma, self.norm_eps = None, 0.0

    def load_canonical(self, w13, w2, w13_sf=None, w2_sf=None, w13_gs=None, w2_gs=None,
                       w2_input_scale=None, stream=None):
        """Canonical device tensors (include/moe.h layout) -> kernel layout."""
        self.w13_k = torch.empty_like(w13)
        self.w2_k = torch.empty_like(w2)
        if w13_sf is not None:
            self.w13_sf_k = torch.empty_like(w13_sf)
            self.w2_sf_k = torch.empty_like(w2_sf)
        _lib.moe_transform_weights(self.fmt, self.num_experts, self.hidden, self.inter, w13, w13_sf, w2, w2_sf,
                                   self.w13_k, self.w13_sf_k, self.w2_k, self.w2_sf_k, stream)
        if self.fmt == "nvfp4":
            self.w13_gs = w13_gs.to(self.device, torch.float32).contiguous()
            self.w2_gs = w2_gs.to(self.device, torch.float32).contiguous()
            # the kernel quantises every L2 input with the max of the experts'
            # w2 input scales (1.0 if that max is 0)
            m = float(w2_input_scale.max()) if w2_input_scale is not None else 0.0
            self.l2_activation_scale = m if m > 0 else 1.0

    def set_post_expert_norm(self, weight, eps, gain_center=None):
        """Post-expert RMSNorm applied by every later ``forward``.  The library
        applies gamma as given, so a zero-centred gain (the stored weight is
        the offset from ``gain_center``) is folded in here, once, as the
        Muse-Spark MegaMoE page's holder does before its kernel runs."""
        gamma = weight.to(self.device, torch.float32)
        if gain_center is not None:
            gamma = gamma + float(gain_center)
        self.norm_gamma, self.norm_eps = gamma.contiguous(), float(eps)

    def forward(self, x, topk_ids, topk_weights, out=None, block_m=0, stream=None, step_events=None,
                norm_gamma=None, norm_eps=None, weight_on_input=False):
        """``norm_gamma`` (float32 [H]) / ``norm_eps``: post-expert RMSNorm of
        the output (default: what ``set_post_expert_norm`` stored, if
        anything); ``weight_on_input``: the routing weight scales the input
        (top_k = 1, no shared expert)."""
        if norm_gamma is None:
            norm_gamma = self.norm_gamma
            norm_eps = self.norm_eps if norm_eps is None else norm_eps
        norm_eps = 0.0 if norm_eps is None else norm_eps
        T = x.shape[0]
        if T > self.max_tokens:
            raise ValueError(f"{T} tokens, but the workspace was sized for {self.max_tokens}")
        if out is None:
            out = torch.empty((T, self.hidden), dtype=torch.bfloat16, device=self.device)
        return _lib.moe_forward(self.fmt, T, self.hidden, self.inter, self.top_k, self.expert_start,
                                self.num_local_experts, self.num_shared, block_m, self.act, x, topk_ids,
                                topk_weights, self.w13_k, self.w13_sf_k, self.w2_k, self.w2_sf_k,
                                self.w13_gs, self.w2_gs, self.l2_activation_scale, out, self.workspace,
                                stream=stream, step_events=step_events, norm_gamma=norm_gamma, norm_eps=norm_eps,
                                weight_on_input=weight_on_input)
