"""Seeded generators.

RNG streams: ``numpy.random.default_rng(SeedSequence([seed, cfg_id,
tensor_id, expert_id]))``.  Tensors: x ~ N(0, x_std) as float32 then BF16
(torch's round-to-nearest-even cast); weights ~ N(0, w_std) as float32 (the
caller casts or quantises); router draws as listed per routing kind.

Large weight sets (billions of elements) are drawn on the device instead
with ``torch.Generator`` seeded from the same tuple: same distribution,
different stream; tests that compare those against the oracle copy the drawn
float32 slices to the host.
"""

import numpy as np
import torch

from .configs import MoEConfig

T_X, T_W13, T_W2, T_ROUTE, T_W2IN = 1, 2, 3, 4, 5


def _rng(cfg: MoEConfig, tensor_id, expert_id=0, seed=0):
    return np.random.default_rng(np.random.SeedSequence([seed, cfg.cfg_id, tensor_id, expert_id]))


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """BF16 torch tensor -> uint16 bit patterns (host NumPy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def gen_x_bf16(cfg: MoEConfig, T=None, seed=0) -> torch.Tensor:
    """x [T, H] ~ N(0, x_std), BF16 (CPU tensor)."""
    T = cfg.T if T is None else T
    x = _rng(cfg, T_X, 0, seed).standard_normal((T, cfg.H), dtype=np.float32)
    x *= np.float32(cfg.x_std)
    return torch.from_numpy(x).to(torch.bfloat16)


def weight_shape(cfg: MoEConfig, which):
    return (2 * cfg.I, cfg.H) if which == "w13" else (cfg.H, cfg.I)


def gen_weight_f32(cfg: MoEConfig, which, e, seed=0) -> np.ndarray:
    """One expert's float32 weight [N, K] ~ N(0, w_std); w13 rows are
    [gate (I rows); up (I rows)].  Experts E .. E+num_shared-1 are the shared
    experts."""
    tid = T_W13 if which == "w13" else T_W2
    w = _rng(cfg, tid, e, seed).standard_normal(weight_shape(cfg, which), dtype=np.float32)
    w *= np.float32(cfg.w_std)
    return w


def _device_seed(cfg, tid, e, seed):
    return int(np.random.SeedSequence([seed, cfg.cfg_id, tid, e, 7]).generate_state(1, np.uint64)[0] >> 1)


def gen_weight_f32_device(cfg: MoEConfig, which, e, device, seed=0) -> torch.Tensor:
    """Device-drawn float32 weight [N, K] ~ N(0, w_std) (torch Philox)."""
    tid = T_W13 if which == "w13" else T_W2
    g = torch.Generator(device=device)
    g.manual_seed(_device_seed(cfg, tid, e, seed))
    w = torch.randn(weight_shape(cfg, which), generator=g, device=device, dtype=torch.float32)
    return w.mul_(cfg.w_std)


def gen_routing(cfg: MoEConfig, T=None, seed=0):
    """-> (topk_ids int32 [T, k], topk_weights float32 [T, k]).

    softmax_normal / softmax_uniform: logits ~ N(0,1) / U[0,1), softmax,
    top-k, renormalised.  sigmoid_normal: logits ~ N(0,1), score = sigmoid,
    top-k by score, weights = score / sum of the chosen scores.  zipf: a seeded
    permutation ranks the experts; logit = -s * ln(rank) + Gumbel(0, 1), so
    the top-k are k draws without replacement with P(e) ~ rank(e)^-s; weights
    are the softmax over the chosen logits.  Ties pick the lower expert id.
    """
    T = cfg.T if T is None else T
    rng = _rng(cfg, T_ROUTE, 0, seed)
    E, k = cfg.E, cfg.top_k
    if cfg.routing == "softmax_normal":
        logits = rng.standard_normal((T, E))
    elif cfg.routing in ("softmax_uniform",):
        logits = rng.random((T, E))
    elif cfg.routing == "sigmoid_normal":
        logits = rng.standard_normal((T, E))
    elif cfg.routing == "zipf":
        perm = rng.permutation(E)
        rank = np.empty(E)
        rank[perm] = np.arange(1, E + 1)
        logits = -cfg.zipf_s * np.log(rank)[None, :] + rng.gumbel(size=(T, E))
    else:
        raise ValueError(cfg.routing)
    if cfg.routing == "sigmoid_normal":
        score = 1.0 / (1.0 + np.exp(-logits))
    else:
        score = logits
    ids = np.argsort(-score, axis=1, kind="stable")[:, :k]
    chosen = np.take_along_axis(score, ids, axis=1)
    if cfg.routing == "sigmoid_normal":
        w = chosen / chosen.sum(axis=1, keepdims=True)
    else:
        z = np.exp(chosen - chosen.max(axis=1, keepdims=True))
        w = z / z.sum(axis=1, keepdims=True)
    return ids.astype(np.int32), w.astype(np.float32)


def gen_w2_input_scale(cfg: MoEConfig, seed=0, amax_nominal=32.0) -> np.ndarray:
    """NVFP4 per-expert L2 input scales [E + num_shared] (a checkpoint
    calibration constant on the pages; synthetic here): U[0.75, 1) times
    amax_nominal / (6 * 448), with amax_nominal above the largest L2 input
    the seeded workloads produce so no block scale saturates."""
    rng = _rng(cfg, T_W2IN, 0, seed)
    u = rng.uniform(0.75, 1.0, cfg.E + cfg.num_shared)
    return (u * amax_nominal / 2688.0).astype(np.float32)
