"""The HIP layer at the full sizes of the five seeded workloads, in the launch
configuration bench.py times (default BLOCK_M), against the oracle on
sampled tokens.

Full-size weight sets are drawn on the device (synth.gen_weight_f32_device)
and, for the MX/NVFP4 formats, quantised by the library.  For the sampled
tokens' experts the oracle re-quantises the same float32 draws with its own
quantiser (in a process pool) and the GPU's codes must match them bit for
bit; the oracle then computes those tokens' outputs from its own codes.
Routing metadata is checked bit-exact at full size.  Bar: as in
tests/helpers.check_layer, with RMS taken over the sampled outputs.
"""

import concurrent.futures
import os
import sys

import numpy as np
import pytest
import torch

import expert_gemms_amd as moe
from oracle import codecs, quant
from oracle.dispatch import dispatch_reference
from oracle.moe import moe_reference
from synth import CONFIGS, gen_routing, gen_w2_input_scale, gen_weight_f32_device, gen_x_bf16, bf16_bits
from synth.configs import DECODE_TOKENS
from tests.gpu_util import dev
from tests.helpers import check_layer

pytestmark = pytest.mark.gpu

CASES = [("tiny_bf16", None), ("mixtral_bf16", None), ("dsv3_mxfp8", None), ("nvfp4_zipf", None)] + \
        [("decode_mxfp4", t) for t in DECODE_TOKENS]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _oracle_quantize(args):
    """(fmt, float32 [N, K]) -> canonical arrays of one expert (oracle side)."""
    fmt, w32 = args
    if fmt == "mxfp8":
        q, c = quant.mx_quantize(w32, "e4m3")
        return {"w": q, "sf": c}
    if fmt == "mxfp4":
        q, c = quant.mx_quantize(w32, "e2m1")
        return {"w": codecs.fp4_pack(q), "sf": c}
    g = quant.nvfp4_global_scale(np.array(np.abs(w32).max(), dtype=np.float32))
    q, bs = quant.nvfp4_quantize(w32, np.full(w32.shape[0], g, dtype=np.float32))
    return {"w": codecs.fp4_pack(q), "sf": bs, "gs": np.float32(g)}


class ExpertArray:
    """Per-expert canonical arrays for the experts the oracle needs."""
    def __init__(self, n_experts, items):
        self.items = items
        self.shape = (n_experts,)

    def __getitem__(self, e):
        return self.items[int(e)]


def pick_tokens(ids, n_tok, E):
    """A few tokens (first one fixed) chosen greedily to share experts, so the
    oracle re-quantises as few experts as possible."""
    T = ids.shape[0]
    chosen = [0]
    experts = set(int(e) for e in ids[0] if 0 <= e < E)
    rng = np.random.default_rng(123)
    cand = rng.permutation(T)[:4096]
    while len(chosen) < min(n_tok, T):
        best, best_new = None, None
        for t in cand:
            if t in chosen:
                continue
            new = len(set(int(e) for e in ids[t] if 0 <= e < E) - experts)
            if best_new is None or new < best_new:
                best, best_new = int(t), new
        chosen.append(best)
        experts |= set(int(e) for e in ids[best] if 0 <= e < E)
    chosen.append(T - 1)
    return sorted(set(chosen))


@pytest.mark.parametrize("name,tokens", CASES, ids=[f"{n}-{t}" if t else n for n, t in CASES])
def test_fullsize_sampled(name, tokens):
    cfg = CONFIGS[name]
    T = tokens if tokens is not None else cfg.T
    fmt, H, I = cfg.fmt, cfg.H, cfg.I
    E_all = cfg.E + cfg.num_shared
    log(f"[fullsize] {name} T={T} fmt={fmt}: inputs")
    x = gen_x_bf16(cfg, T)
    ids, wts = gen_routing(cfg, T)
    bm = moe.moe_get_block_m(T, cfg.E, cfg.num_shared, cfg.top_k, fmt)

    # routing metadata at full size, bit-exact
    S = T * (cfg.top_k + cfg.num_shared)
    M = S + E_all * (bm - 1)
    d = lambda n: torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
    cnt, off, ss, sr, te = d(E_all), d(E_all + 1), d(M), d(S), d(M // bm + 1)
    ids_d = dev(ids)
    # with the scratch moe_forward's workspace provides (many workgroups from
    # 16384 slots on, as in the forward)
    bc = d(moe._lib.dispatch_scratch_ints(T, cfg.top_k, cfg.num_shared, cfg.E))
    moe.moe_dispatch(T, cfg.top_k, cfg.num_shared, 0, cfg.E, bm, ids_d, cnt, off, ss, sr, te, block_counts=bc)
    ref_d = dispatch_reference(ids, cfg.num_shared, 0, cfg.E, bm)
    Mp = int(ref_d["offsets"][-1])
    got = {"counts": cnt.cpu().numpy()[:E_all], "offsets": off.cpu().numpy(), "sorted_slot": ss.cpu().numpy()[:Mp],
           "slot_row": sr.cpu().numpy()[:S], "tile_expert": te.cpu().numpy()[:Mp // bm]}
    for k in ref_d:
        assert np.array_equal(got[k], ref_d[k]), k
    log(f"[fullsize] {name}: dispatch bit-exact (BLOCK_M {bm}, {Mp} padded rows)")

    sample = pick_tokens(ids, 3 if fmt != "bf16" else 6, cfg.E)
    needed = sorted(set(int(e) for t in sample for e in ids[t] if 0 <= e < cfg.E) |
                    set(range(cfg.E, E_all)))
    log(f"[fullsize] {name}: sampled tokens {sample}, {len(needed)} experts for the oracle")

    # weights: drawn on the device, quantised by the library
    vpe = 2 if fmt in ("mxfp4", "nvfp4") else 1
    grp = 16 if fmt == "nvfp4" else 32
    canon, host32 = {}, {"w13": {}, "w2": {}}
    for nm, (N, K) in (("w13", (2 * I, H)), ("w2", (H, I))):
        if fmt == "bf16":
            wt = torch.empty((E_all, N, K), dtype=torch.bfloat16, device="cuda")
        else:
            wt = torch.empty((E_all, N, K // vpe), dtype=torch.uint8, device="cuda")
            sf = torch.empty((E_all, N, K // grp), dtype=torch.uint8, device="cuda")
            gs = torch.empty((E_all,), dtype=torch.float32, device="cuda") if fmt == "nvfp4" else None
        for e in range(E_all):
            src = gen_weight_f32_device(cfg, nm, e, "cuda")
            if e in needed:
                host32[nm][e] = src.cpu().numpy()
            if fmt == "bf16":
                wt[e].copy_(src)
            else:
                moe.moe_quantize_weights(fmt, 1, N, K, src, wt[e], sf[e], gs[e:e + 1] if gs is not None else None)
        canon[nm] = wt
        if fmt != "bf16":
            canon[nm + "_sf"] = sf
            if gs is not None:
                canon[nm + "_gs"] = gs
    torch.cuda.synchronize()
    log(f"[fullsize] {name}: weights ready")

    layer = moe.FusedMoE(fmt, H, I, cfg.E, cfg.top_k, num_shared=cfg.num_shared, max_tokens=T)
    w2in = gen_w2_input_scale(cfg) if fmt == "nvfp4" else None
    layer.load_canonical(canon["w13"], canon["w2"], canon.get("w13_sf"), canon.get("w2_sf"),
                         canon.get("w13_gs"), canon.get("w2_gs"),
                         w2_input_scale=None if w2in is None else torch.from_numpy(w2in))
    y = layer.forward(x.cuda(), ids_d, dev(wts))
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    log(f"[fullsize] {name}: GPU forward done")

    # oracle-side canonical arrays of the needed experts, checked against the GPU's
    w = {}
    if fmt == "bf16":
        for nm in ("w13", "w2"):
            items = {e: bf16_bits(torch.from_numpy(host32[nm][e]).to(torch.bfloat16)) for e in needed}
            w[nm] = ExpertArray(E_all, items)
    else:
        with concurrent.futures.ProcessPoolExecutor(max_workers=8) as ex:
            for nm in ("w13", "w2"):
                res = dict(zip(needed, ex.map(_oracle_quantize, [(fmt, host32[nm][e]) for e in needed])))
                for e in needed:
                    assert np.array_equal(canon[nm][e].cpu().numpy(), res[e]["w"]), (nm, e)
                    assert np.array_equal(canon[nm + "_sf"][e].cpu().numpy(), res[e]["sf"]), (nm, e)
                    if fmt == "nvfp4":
                        assert canon[nm + "_gs"][e].item() == res[e]["gs"], (nm, e)
                w[nm] = ExpertArray(E_all, {e: res[e]["w"] for e in needed})
                w[nm + "_sf"] = ExpertArray(E_all, {e: res[e]["sf"] for e in needed})
                if fmt == "nvfp4":
                    gsv = np.zeros(E_all, dtype=np.float32)
                    for e in needed:
                        gsv[e] = res[e]["gs"]
                    w[nm + "_gs"] = gsv
        log(f"[fullsize] {name}: GPU weight codes equal the oracle's for {len(needed)} experts")
    g2 = 1.0
    if fmt == "nvfp4":
        m = float(w2in.max())
        g2 = m if m > 0 else 1.0
    ref = moe_reference(fmt, bf16_bits(x), ids, wts, w, num_shared=cfg.num_shared, tokens=sample,
                        l2_activation_scale=g2)
    rel, excess, alt = check_layer(fmt, y[sample], ref, bf16_bits(x), ids, wts, w, num_shared=cfg.num_shared,
                                   g2=g2, tokens=sample)
    log(f"[fullsize] {name}: sampled max|err|/RMS = {rel:.3e}; tokens under another valid L2-input decision: {alt}")
    assert excess <= 0, (rel, excess)
    assert np.isfinite(y).all()
