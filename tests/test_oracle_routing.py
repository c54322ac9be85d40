"""Pins of the router top-k oracle (CPU)."""

import numpy as np
import pytest
import torch

from oracle.routing import kept_experts, route_reference, scores_of


def brute_force(logits, top_k, scoring, bias, num_groups, topk_groups, renormalize, scaling):
    """Nested loops: pick the best remaining expert k times (ties to the lower
    id) among the experts of the best groups (group rank: its best expert)."""
    T, E = logits.shape
    ids = np.zeros((T, top_k), dtype=np.int32)
    w = np.zeros((T, top_k))
    for t in range(T):
        if scoring == "softmax":
            m = max(logits[t])
            ex = [np.exp(v - m) for v in logits[t]]
            sc = [v / sum(ex) for v in ex]
        else:
            sc = [1.0 / (1.0 + np.exp(-v)) for v in logits[t]]
        ch = [sc[e] + (bias[e] if bias is not None else 0.0) for e in range(E)]
        allowed = set(range(E))
        if num_groups > 1:
            gs = E // num_groups
            gbest = [max(ch[g * gs:(g + 1) * gs]) for g in range(num_groups)]
            kept = []
            for _ in range(topk_groups):
                best = None
                for g in range(num_groups):
                    if g not in kept and (best is None or gbest[g] > gbest[best]):
                        best = g
                kept.append(best)
            allowed = {e for e in range(E) if e // gs in kept}
        chosen = []
        for _ in range(top_k):
            best = None
            for e in range(E):
                if e in allowed and e not in chosen and (best is None or ch[e] > ch[best]):
                    best = e
            chosen.append(best)
        ids[t] = chosen
        ws = [sc[e] for e in chosen]
        if renormalize:
            ws = [v / sum(ws) for v in ws]
        w[t] = [v * scaling for v in ws]
    return ids, w


CASES = [
    dict(scoring="softmax", bias=False, num_groups=1, topk_groups=1, renormalize=True, scaling=1.0),
    dict(scoring="softmax", bias=False, num_groups=1, topk_groups=1, renormalize=False, scaling=1.0),
    dict(scoring="sigmoid", bias=True, num_groups=4, topk_groups=2, renormalize=True, scaling=2.5),
    dict(scoring="softmax", bias=True, num_groups=1, topk_groups=1, renormalize=True, scaling=1.5),
    dict(scoring="sigmoid", bias=False, num_groups=8, topk_groups=3, renormalize=False, scaling=1.0),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_matches_brute_force(case):
    c = CASES[case]
    rng = np.random.default_rng(case)
    T, E, k = 7, 16, 4
    # coarse values so exact ties occur
    logits = np.round(rng.standard_normal((T, E)) * 4) / 4
    bias = np.round(rng.standard_normal(E) * 8) / 64 if c["bias"] else None
    ids, w, _ = route_reference(logits, k, scoring=c["scoring"], bias=bias, num_groups=c["num_groups"],
                                topk_groups=c["topk_groups"], renormalize=c["renormalize"], scaling=c["scaling"])
    bids, bw = brute_force(logits, k, c["scoring"], bias, c["num_groups"], c["topk_groups"], c["renormalize"],
                           c["scaling"])
    assert np.array_equal(ids, bids)
    assert np.allclose(w, bw, rtol=1e-12, atol=0)


def test_against_torch_stable_sort():
    """Plain top-k equals torch's stable descending sort of the softmax."""
    rng = np.random.default_rng(5)
    logits = np.round(rng.standard_normal((50, 64)) * 3) / 3
    ids, w, _ = route_reference(logits, 6, renormalize=False)
    p = torch.softmax(torch.from_numpy(logits), dim=-1)
    order = torch.sort(p, dim=-1, descending=True, stable=True).indices[:, :6].numpy()
    assert np.array_equal(ids, order)
    assert np.allclose(w, torch.gather(p, 1, torch.from_numpy(order).long()).numpy(), rtol=1e-12)


def test_closed_forms():
    logits = np.array([[0.0, np.log(3.0), np.log(2.0), np.log(2.0)]])
    s = scores_of(logits, "softmax")
    assert np.allclose(s, [[1 / 8, 3 / 8, 2 / 8, 2 / 8]])
    ids, w, _ = route_reference(logits, 2, renormalize=True)
    assert ids.tolist() == [[1, 2]]                      # tie between 2 and 3 goes to 2
    assert np.allclose(w, [[3 / 5, 2 / 5]])
    assert np.allclose(scores_of(np.array([[0.0, 2.0]]), "sigmoid") + scores_of(np.array([[0.0, -2.0]]), "sigmoid"),
                       [[1.0, 1.0]])


def test_bias_moves_choice_not_weights():
    logits = np.array([[1.0, 0.9, 0.0, -1.0]])
    bias = np.array([0.0, 0.0, 0.5, 0.0])
    ids, w, _ = route_reference(logits, 2, scoring="sigmoid", bias=bias, renormalize=False)
    s = scores_of(logits, "sigmoid")[0]
    assert ids.tolist() == [[2, 0]]                      # 0.5 + 0.5 before 0.731
    assert np.allclose(w, [[s[2], s[0]]])


def test_groups_and_special_cases():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((20, 32))
    base, _, _ = route_reference(logits, 4, scoring="sigmoid", num_groups=1)
    all_groups, _, _ = route_reference(logits, 4, scoring="sigmoid", num_groups=8, topk_groups=8)
    assert np.array_equal(base, all_groups)              # keeping every group changes nothing
    ids, _, _ = route_reference(logits, 4, scoring="sigmoid", num_groups=8, topk_groups=2)
    keep = kept_experts(scores_of(logits, "sigmoid"), 8, 2)
    assert np.take_along_axis(keep, ids.astype(np.int64), axis=1).all()
    _, w, _ = route_reference(logits, 5, renormalize=True, scaling=2.5)
    assert np.allclose(w.sum(axis=1), 2.5)
    ids, _, _ = route_reference(logits, 32)
    assert (np.sort(ids, axis=1) == np.arange(32)).all()
    pad = np.zeros(20, dtype=bool)
    pad[[3, 7]] = True
    ids, w, _ = route_reference(logits, 4, is_padding=pad)
    assert (ids[pad] == -1).all() and (w[pad] == 0).all() and (ids[~pad] >= 0).all()
