"""Routing metadata of the grouped GEMMs (oracle side).

Sources on the pages:

* "fused_moe" package page, ``DeepGemmExperts.apply``: the contiguous layout
  pads every expert's group of rows to the GEMM's M alignment
  (``compute_aligned_M``), permutes token rows into those groups, and
  un-permutes and reduces after the second GEMM.
* "DeepGEMM MegaMoE experts" page: ``get_block_m`` is the BLOCK_M the
  scheduler pads groups to; a rank owns the physical experts
  ``[experts_start_idx, experts_start_idx + num_local_experts)``; a fused
  shared expert is always selected.

Readings: a slot is one (token, choice) pair, flat index ``t * k' + j`` with
``k' = top_k + num_shared``; shared slots come after the routed ones and use
the local experts ``num_local .. num_local + num_shared - 1``; routed ids
outside the local range (including -1) are dropped; within an expert's group
slots keep ascending flat order (a stable sort), padding rows are -1, and an
expert with no slots gets no rows.
"""

import numpy as np


def slot_experts(topk_ids, num_shared, expert_start, num_local):
    """Local expert of every slot, -1 for a dropped slot.  [T, k'] int64."""
    ids = np.asarray(topk_ids, dtype=np.int64)
    T, k = ids.shape
    loc = ids - expert_start
    routed = np.where((loc >= 0) & (loc < num_local), loc, -1)
    shared = np.broadcast_to(num_local + np.arange(num_shared, dtype=np.int64),
                             (T, num_shared))
    return np.concatenate([routed, shared], axis=1)


def dispatch_reference(topk_ids, num_shared, expert_start, num_local, block_m):
    """Returns a dict of int32 arrays:

    counts[E'], offsets[E'+1] (exclusive scan of counts rounded up to
    ``block_m``), sorted_slot[M_pad] (flat slot ids grouped by expert in
    ascending order, -1 for padding), slot_row[S] (row of each slot in the
    sorted order, -1 if dropped), tile_expert[M_pad / block_m].
    """
    exp = slot_experts(topk_ids, num_shared, expert_start, num_local).reshape(-1)
    E = num_local + num_shared
    S = exp.size
    counts = np.bincount(exp[exp >= 0], minlength=E).astype(np.int64)
    padded = -(-counts // block_m) * block_m
    offsets = np.concatenate([[0], np.cumsum(padded)]).astype(np.int64)
    M_pad = int(offsets[-1])
    sorted_slot = np.full(M_pad, -1, dtype=np.int64)
    slot_row = np.full(S, -1, dtype=np.int64)
    order = np.argsort(exp, kind="stable")
    order = order[exp[order] >= 0]
    pos = 0
    for e in range(E):
        n = int(counts[e])
        slots = order[pos:pos + n]
        pos += n
        rows = offsets[e] + np.arange(n)
        sorted_slot[rows] = slots
        slot_row[slots] = rows
    tile_expert = np.repeat(np.arange(E), padded // block_m)
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "sorted_slot": sorted_slot.astype(np.int32),
        "slot_row": slot_row.astype(np.int32),
        "tile_expert": tile_expert.astype(np.int32),
    }

