"""The HIP layer at the full sizes of the five seeded workloads, in the launch
configuration bench.py times (the library's BLOCK_M and K-split rules),
against the oracle over whole outputs.

Weights: each expert's float32 draws (synth.gen_weight_f32) are quantised by
the oracle's quantisers (tests/helpers.quantize_weight) in a process pool;
the same canonical arrays go to the GPU (moe_transform_weights) and to the
oracle, so no oracle input comes from the HIP path.

Compared: every token of the Mixtral-shaped BF16 layer, the NVFP4 Zipf layer
and every decode batch, and 256 tokens of the DeepSeek-V3-shaped layer
(nearly every one of its 257 experts); the oracle's output is the sum of
per-expert-group contributions computed in the pool (the layer is a sum over
slots; the shared expert enters as an always-present id of weight 1).  Also
checked from the forward's own workspace: the routing metadata and the
dispatch-quantised x bit-exact at full size, and the L2-input codes of the
first 64 compared tokens (16 for the DeepSeek-V3 layer) against the
oracle's quantiser.
"""

import concurrent.futures
import multiprocessing
import os
import sys
import time

import numpy as np
import pytest
import torch

import expert_gemms_amd as moe
from oracle import codecs, quant
from oracle.dispatch import dispatch_reference
from oracle.moe import moe_reference
from synth import CONFIGS, gen_routing, gen_w2_input_scale, gen_weight_f32, gen_x_bf16, bf16_bits
from synth.configs import DECODE_TOKENS
from tests.gpu_util import WorkspaceReader, dev
from tests.helpers import (check_layer, l2_code_check, quantize_weight, record_parity, rescue_cap,
                           slot_l2_inputs)

pytestmark = pytest.mark.gpu

CASES = [("tiny_bf16", None), ("mixtral_bf16", None), ("dsv3_mxfp8", None), ("nvfp4_zipf", None)] + \
        [("decode_mxfp4", t) for t in DECODE_TOKENS]
COMPARED_TOKENS = {"dsv3_mxfp8": 256}
L2_CHECK_TOKENS = {"dsv3_mxfp8": 16}      # else 64
WORKERS = min(16, os.cpu_count() or 1)


def log(msg):
    print(f"[fullsize {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def _limit_blas():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(2)
    except Exception:
        pass


def _expert_weights(args):
    """(workload, expert) -> canonical arrays of that expert (oracle side)."""
    name, e = args
    cfg = CONFIGS[name]
    return e, {nm: quantize_weight(cfg.fmt, gen_weight_f32(cfg, nm, e)) for nm in ("w13", "w2")}


class ExpertArray:
    """Per-expert canonical arrays indexed like the stacked [E', ...] array."""
    def __init__(self, n_experts, items):
        self.items = items
        self.shape = (n_experts,)

    def __getitem__(self, e):
        return self.items[int(e)]


def _as_w(fmt, n_experts, per_expert):
    w = {}
    for nm in ("w13", "w2"):
        w[nm] = ExpertArray(n_experts, {e: d[nm]["w"] for e, d in per_expert.items()})
        if fmt != "bf16":
            w[nm + "_sf"] = ExpertArray(n_experts, {e: d[nm]["sf"] for e, d in per_expert.items()})
        if fmt == "nvfp4":
            gs = np.zeros(n_experts, dtype=np.float32)
            for e, d in per_expert.items():
                gs[e] = d[nm]["gs"]
            w[nm + "_gs"] = gs
    return w


def _oracle_part(args):
    """The oracle's contribution of one group of experts to the compared
    tokens, and (for the first tokens) the activations entering the L2-input
    quantiser with their error bounds.  The canonical arrays come from the
    parent's memory (a forked worker)."""
    name, group, x_bits, ids_aug, wts_aug, g2, l2_tokens = args
    cfg = CONFIGS[name]
    fmt, n_experts = cfg.fmt, cfg.E + cfg.num_shared
    per_expert = {e: _WEIGHTS[name][e] for e in group}
    w = _as_w(fmt, n_experts, per_expert)
    mine = np.isin(ids_aug, list(per_expert))
    ids_m = np.where(mine, ids_aug, -1)
    y = moe_reference(fmt, x_bits, ids_m, wts_aug, w, num_shared=0, num_local=n_experts,
                      l2_activation_scale=g2)
    l2 = slot_l2_inputs(fmt, x_bits[:l2_tokens], ids_m[:l2_tokens], w, num_shared=0, num_local=n_experts)
    return y, l2


_WEIGHTS = {}


def oracle_weights(name, pool):
    """Canonical arrays of every expert of a workload (cached: the decode
    batches share one weight set)."""
    if name not in _WEIGHTS:
        cfg = CONFIGS[name]
        E_all = cfg.E + cfg.num_shared
        _WEIGHTS.clear()
        got = {}
        for e, d in pool.map(_expert_weights, [(name, e) for e in range(E_all)]):
            got[e] = d
            if len(got) % 16 == 0:
                log(f"{name}: {len(got)} of {E_all} experts quantised")
        _WEIGHTS[name] = got
    return _WEIGHTS[name]


def upload(fmt, per_expert, E_all):
    """Stacked canonical device tensors."""
    out = {}
    for nm in ("w13", "w2"):
        out[nm] = dev(np.stack([per_expert[e][nm]["w"] for e in range(E_all)]))
        if fmt != "bf16":
            out[nm + "_sf"] = dev(np.stack([per_expert[e][nm]["sf"] for e in range(E_all)]))
        if fmt == "nvfp4":
            out[nm + "_gs"] = dev(np.array([per_expert[e][nm]["gs"] for e in range(E_all)], dtype=np.float32))
    return out


def compared_tokens(name, ids, T, E):
    """All tokens, or for the largest layer a set chosen greedily to reach
    as many (expert, first-seen) pairs as possible: each next token adds the
    most experts not yet covered."""
    n = COMPARED_TOKENS.get(name)
    if n is None or n >= T:
        return np.arange(T)
    rng = np.random.default_rng(321)
    cand = rng.permutation(T)[:4 * n]
    chosen, seen = [], set()
    left = list(cand)
    while len(chosen) < n:
        gains = [len(set(int(e) for e in ids[t] if 0 <= e < E) - seen) for t in left]
        i = int(np.argmax(gains))
        t = left.pop(i)
        chosen.append(int(t))
        seen |= set(int(e) for e in ids[t] if 0 <= e < E)
    return np.array(sorted(chosen))


def expert_groups(counts, n_groups):
    """Experts split into groups of about equal slot counts (largest first)."""
    order = np.argsort(-counts, kind="stable")
    groups = [[] for _ in range(n_groups)]
    load = np.zeros(n_groups)
    for e in order:
        if counts[e] == 0:
            continue
        g = int(np.argmin(load))
        groups[g].append(int(e))
        load[g] += counts[e] + 1
    return [g for g in groups if g]


@pytest.mark.parametrize("name,tokens", CASES, ids=[f"{n}-{t}" if t else n for n, t in CASES])
def test_fullsize(name, tokens):
    cfg = CONFIGS[name]
    T = tokens if tokens is not None else cfg.T
    fmt, H, I = cfg.fmt, cfg.H, cfg.I
    E_all = cfg.E + cfg.num_shared
    kk = cfg.top_k + cfg.num_shared
    log(f"{name} T={T} fmt={fmt}: inputs")
    x = gen_x_bf16(cfg, T)
    xb = bf16_bits(x)
    ids, wts = gen_routing(cfg, T)
    fork = multiprocessing.get_context("fork")
    with concurrent.futures.ProcessPoolExecutor(max_workers=WORKERS, initializer=_limit_blas,
                                                mp_context=fork) as pool:
        per_expert = oracle_weights(name, pool)
    log(f"{name}: {E_all} experts quantised by the oracle's quantisers")
    # a pool forked now sees the canonical arrays without copying them over
    with concurrent.futures.ProcessPoolExecutor(max_workers=WORKERS, initializer=_limit_blas,
                                                mp_context=fork) as pool:

        # the GPU forward, default BLOCK_M and K splits
        canon = upload(fmt, per_expert, E_all)
        layer = moe.FusedMoE(fmt, H, I, cfg.E, cfg.top_k, num_shared=cfg.num_shared, max_tokens=T)
        w2in = gen_w2_input_scale(cfg) if fmt == "nvfp4" else None
        layer.load_canonical(canon["w13"], canon["w2"], canon.get("w13_sf"), canon.get("w2_sf"),
                             canon.get("w13_gs"), canon.get("w2_gs"),
                             w2_input_scale=None if w2in is None else torch.from_numpy(w2in))
        y = layer.forward(x.cuda(), dev(ids), dev(wts))
        torch.cuda.synchronize()
        y = y.float().cpu().numpy().astype(np.float64)
        del canon
        ws = WorkspaceReader(layer, T)
        log(f"{name}: GPU forward done (BLOCK_M {ws.bm}, L1 split {ws.lay['l1_ksplit']}, "
            f"L2 split {ws.lay['l2_ksplit']})")

        # routing metadata and dispatch-quantised x of the forward, bit-exact
        ref_d = dispatch_reference(ids, cfg.num_shared, 0, cfg.E, ws.bm)
        got = ws.dispatch()
        for k in ref_d:
            assert np.array_equal(got[k], ref_d[k]), k
        if fmt != "bf16":
            x32 = codecs.bf16_decode(xb).astype(np.float32)
            codes, scales, tok = ws.xq()
            if fmt == "nvfp4":
                g = quant.nvfp4_global_scale(np.abs(x32).max(axis=1))
                q, bs = quant.nvfp4_quantize(x32, g)
                assert np.array_equal(tok, g)
            else:
                q, bs = quant.mx_quantize(x32, "e4m3")
            assert np.array_equal(codes, q) and np.array_equal(scales, bs)
        log(f"{name}: dispatch and dispatch quantisation bit-exact ({int(ref_d['offsets'][-1])} padded rows)")

        # the oracle over the compared tokens, by groups of experts
        sample = compared_tokens(name, ids, T, cfg.E)
        ids_aug = np.concatenate([ids[sample].astype(np.int64),
                                  np.broadcast_to(cfg.E + np.arange(cfg.num_shared), (sample.size, cfg.num_shared))],
                                 axis=1)
        wts_aug = np.concatenate([wts[sample].astype(np.float64), np.ones((sample.size, cfg.num_shared))], axis=1)
        counts = np.bincount(ids_aug[ids_aug >= 0].ravel(), minlength=E_all)
        groups = expert_groups(counts, min(WORKERS * 2, E_all))
        g2 = 1.0
        if fmt == "nvfp4":
            m = float(w2in.max())
            g2 = m if m > 0 else 1.0
        l2_tokens = min(L2_CHECK_TOKENS.get(name, 64), sample.size)
        jobs = [(name, grp, xb[sample], ids_aug, wts_aug, g2, l2_tokens) for grp in groups]
        ref = np.zeros((sample.size, H))
        l2_parts = []
        for i, (part, l2) in enumerate(pool.map(_oracle_part, jobs)):
            ref += part
            l2_parts.append(l2)
            if (i + 1) % 8 == 0:
                log(f"{name}: oracle, {i + 1} of {len(jobs)} expert groups")
    log(f"{name}: oracle done on {sample.size} tokens over {len(groups)} expert groups")

    # the layer output
    w = _as_w(fmt, E_all, per_expert)
    rel, excess, alt = check_layer(fmt, y[sample], ref, xb[sample], ids_aug, wts_aug, w, num_shared=0,
                                   num_local=E_all, g2=g2, name=f"fullsize {name} T={T}")
    log(f"{name}: max|err|/RMS = {rel:.3e} over {sample.size} tokens; "
        f"tokens under another valid L2-input decision: {alt}")
    assert excess <= 0, (rel, excess)
    assert alt <= rescue_cap(sample.size), alt
    assert np.isfinite(y).all()

    # L2-input codes of the first compared tokens (slot ids of the augmented
    # routing map back to the forward's slots: same token order, k' columns)
    slots = np.concatenate([p[0] for p in l2_parts])
    a = np.concatenate([p[2] for p in l2_parts])
    da = np.concatenate([p[3] for p in l2_parts])
    fwd_slots = sample[slots // kk] * kk + slots % kk
    rows = got["slot_row"][fwd_slots]
    assert (rows >= 0).all()
    codes, scales = ws.l2_input(rows)
    st = l2_code_check(fmt, codes, scales, a, da, g2=g2)
    record_parity(f"fullsize L2 input {name} T={T} ({l2_tokens} tokens)", **st)
    log(f"{name}: L2-input codes {st}")
    assert st["unexplained"] == 0, st
    cap = 5e-3 if fmt in ("mxfp8", "mxfp4") else 1e-3      # as in tests/test_gpu_workspace.py
    assert st["element_flips"] <= max(2, cap * st["elements"]), st
