"""Router top-k (oracle side): router logits -> (topk_ids, topk_weights).

What is computed follows the "fused_moe" page: ``FusedMoE.select_experts``
routes with ``fused_topk`` (softmax scores, top-k, optional renormalisation),
``fused_topk_bias`` (a per-expert ``e_score_correction_bias``, then the
weights times ``routed_scaling_factor``) or ``grouped_topk`` (experts in
``num_expert_group`` groups of which ``topk_group`` are kept; ``scoring_func``
softmax or sigmoid; bias and scaling factor as above).  The Qwen4-Exp page
routes with ``fused_topk(hidden_states, router_logits, top_k, renormalize)``.
The DeepGEMM MegaMoE experts page's forward takes padding tokens out
(``is_padding``).

The pages name these steps but print no implementation; the readings taken
(each listed in the design doc):

* scores: softmax over all experts of the token, or the logistic sigmoid of
  each logit;
* the correction bias only shifts the scores the choice is made on; the
  weights are the unbiased scores of the chosen experts;
* groups are ``num_groups`` contiguous runs of experts; a group's rank is the
  largest choice score in it; the ``topk_groups`` best groups are kept;
* the top-k among the kept experts by choice score, ties to the lower expert
  id, listed best first (groups likewise, ties to the lower group);
* renormalise: weights divided by their sum; then times the scaling factor;
* a padding token gets ids -1 and weights 0 (every slot dropped).

float64 throughout (the choice is made on float64 scores).
"""

import numpy as np


def scores_of(logits, scoring):
    """float64 scores [T, E] from router logits."""
    x = np.asarray(logits, dtype=np.float64)
    if scoring == "softmax":
        z = np.exp(x - x.max(axis=-1, keepdims=True))
        return z / z.sum(axis=-1, keepdims=True)
    if scoring == "sigmoid":
        return 1.0 / (1.0 + np.exp(-x))
    raise ValueError(scoring)


def kept_experts(choice, num_groups, topk_groups):
    """bool [T, E]: experts in the ``topk_groups`` best groups of each token."""
    T, E = choice.shape
    if num_groups <= 1:
        return np.ones((T, E), dtype=bool)
    gs = E // num_groups
    gscore = choice.reshape(T, num_groups, gs).max(axis=-1)
    order = np.argsort(-gscore, axis=-1, kind="stable")[:, :topk_groups]
    keep_g = np.zeros((T, num_groups), dtype=bool)
    np.put_along_axis(keep_g, order, True, axis=-1)
    return np.repeat(keep_g, gs, axis=-1)


def route_reference(logits, top_k, *, scoring="softmax", bias=None, num_groups=1, topk_groups=1,
                    renormalize=True, scaling=1.0, is_padding=None):
    """-> (ids int32 [T, top_k], weights float64 [T, top_k], choice float64 [T, E])."""
    s = scores_of(logits, scoring)
    choice = s + (0.0 if bias is None else np.asarray(bias, dtype=np.float64)[None, :])
    keep = kept_experts(choice, num_groups, topk_groups)
    masked = np.where(keep, choice, -np.inf)
    ids = np.argsort(-masked, axis=-1, kind="stable")[:, :top_k]
    w = np.take_along_axis(s, ids, axis=-1)
    if renormalize:
        w = w / w.sum(axis=-1, keepdims=True)
    w = w * scaling
    ids = ids.astype(np.int32)
    if is_padding is not None:
        pad = np.asarray(is_padding, dtype=bool)
        ids[pad] = -1
        w[pad] = 0.0
    return ids, w, masked
