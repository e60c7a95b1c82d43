"""Reference token-to-expert sort and padding for the indexed MoE path.  TEST INFRASTRUCTURE ONLY.

"Humming" (wiki article), "Device and workload selection": in the index-routed MoE
form each activation row is fetched by way of the routing table.  The page says no more, so every rule
below is a reading (each is listed in the design notes).  Stability makes the
result unique, so the GPU output must equal it byte for byte.

Inputs: ``topk_ids`` int32 [T, topk]; flat index f = t*topk + j.  E experts, block size BM.

1. cnt[e] = number of f with ids[f] == e (ids outside [0, E) are dropped).
2. pad[e] = ceil(cnt[e] / BM) * BM (empty experts get no block).
3. off[e] = exclusive prefix sum of pad in ascending e.
4. sorted_ids[off[e] + i] = the i-th smallest f routed to e (stable, ascending f);
   sorted_ids[off[e] + cnt[e] .. off[e] + pad[e] - 1] = sentinel T*topk.
5. expert_ids[b] = e for every block b in [off[e]/BM, (off[e] + pad[e])/BM).
6. num_post_pad = sum(pad).
7. Up to capacity: sorted_ids = sentinel, expert_ids = -1.

Capacity (worst case over all routings with the given T, topk, E, BM):
cap_sorted = roundup(T*topk + min(E, T*topk) * (BM - 1), BM), cap_blocks = cap_sorted / BM.
"""
from __future__ import annotations

import numpy as np


def capacity(t: int, topk: int, experts: int, block_m: int):
    tk = t * topk
    raw = tk + min(experts, tk) * (block_m - 1)
    cap_sorted = (raw + block_m - 1) // block_m * block_m
    return cap_sorted, cap_sorted // block_m


def moe_align(topk_ids, experts: int, block_m: int):
    """Vectorised reference (counting sort).  Returns (sorted_ids, expert_ids, num_post_pad)."""
    ids = np.asarray(topk_ids, dtype=np.int64).reshape(-1)
    tk = ids.size
    t, topk = np.asarray(topk_ids).shape
    cap_sorted, cap_blocks = capacity(t, topk, experts, block_m)
    valid = (ids >= 0) & (ids < experts)
    cnt = np.bincount(ids[valid], minlength=experts)[:experts]
    pad = (cnt + block_m - 1) // block_m * block_m
    off = np.concatenate([[0], np.cumsum(pad)[:-1]])
    sorted_ids = np.full(cap_sorted, tk, dtype=np.int32)
    expert_ids = np.full(cap_blocks, -1, dtype=np.int32)
    for e in range(experts):
        f = np.nonzero(ids == e)[0]          # ascending f: the stable order
        sorted_ids[off[e]:off[e] + f.size] = f
        expert_ids[off[e] // block_m:(off[e] + pad[e]) // block_m] = e
    return sorted_ids, expert_ids, int(pad.sum())


def moe_align_bruteforce(topk_ids, experts: int, block_m: int):
    """Pure-Python loops, for pinning the vectorised version on tiny inputs."""
    t, topk = np.asarray(topk_ids).shape
    flat = [int(v) for v in np.asarray(topk_ids).reshape(-1)]
    tk = len(flat)
    cap_sorted, cap_blocks = capacity(t, topk, experts, block_m)
    sorted_ids = [tk] * cap_sorted
    expert_ids = [-1] * cap_blocks
    pos = 0
    for e in range(experts):
        mine = [f for f in range(tk) if flat[f] == e]
        if not mine:
            continue
        nblk = -(-len(mine) // block_m)
        for i, f in enumerate(mine):
            sorted_ids[pos + i] = f
        for b in range(nblk):
            expert_ids[pos // block_m + b] = e
        pos += nblk * block_m
    return np.array(sorted_ids, np.int32), np.array(expert_ids, np.int32), pos


# ---------------------------------------------------------------------------------------
# Grouped MoE input organizations ("Humming" wiki article, "Device and workload selection":
# grouped-contiguous execution keeps each expert's rows together; grouped-masked execution
# gives each expert its own storage with a count of valid rows).  Both name input rows
# directly, so their block map is the contract above applied to one expert id per row
# (topk = 1, flat index = row index):
#   contiguous: rows [offsets[e], offsets[e+1]) belong to expert e; rows_total = offsets[E];
#   masked:     row e*cap + i belongs to expert e for i < counts[e] (counts clamped to
#               [0, cap]); the other rows of the storage are not used; rows_total = E*cap.
# The sentinel is rows_total.

def grouped_row_experts(layout: str, arr, experts: int, cap: int = 0) -> np.ndarray:
    """Expert id of every input row (-1: unused row), int64 [rows_total]."""
    a = np.asarray(arr, dtype=np.int64)
    if layout == "contiguous":
        assert a.size == experts + 1 and a[0] == 0 and np.all(np.diff(a) >= 0)
        return np.repeat(np.arange(experts), np.diff(a))
    assert layout == "masked" and a.size == experts
    cnt = np.clip(a, 0, cap)
    i = np.arange(cap)[None, :]
    return np.where(i < cnt[:, None], np.arange(experts)[:, None], -1).reshape(-1)


def grouped_map(layout: str, arr, experts: int, block_m: int, cap: int = 0, rows_total: int | None = None):
    """(sorted_ids, expert_ids, num_post_pad) of a grouped organization, with the indexed path's
    capacity for rows_total rows and topk = 1.  Contiguous: rows_total defaults to offsets[E];
    rows past offsets[E] belong to no expert."""
    ids = grouped_row_experts(layout, arr, experts, cap)
    if rows_total is not None and rows_total > ids.size:
        ids = np.concatenate([ids, np.full(rows_total - ids.size, -1, dtype=ids.dtype)])
    return moe_align(ids.reshape(-1, 1), experts, block_m)


def grouped_map_direct(layout: str, arr, experts: int, block_m: int, cap: int = 0, rows_total: int | None = None):
    """The same map written out expert by expert with loops, for pinning grouped_map."""
    a = [int(v) for v in np.asarray(arr).reshape(-1)]
    total = (a[experts] if rows_total is None else rows_total) if layout == "contiguous" else experts * cap
    cs, cb = capacity(total, 1, experts, block_m)
    sorted_ids = [total] * cs
    expert_ids = [-1] * cb
    pos = 0
    for e in range(experts):
        if layout == "contiguous":
            rows = list(range(a[e], a[e + 1]))
        else:
            rows = [e * cap + i for i in range(min(max(a[e], 0), cap))]
        if not rows:
            continue
        nblk = -(-len(rows) // block_m)
        sorted_ids[pos:pos + len(rows)] = rows
        for b in range(nblk):
            expert_ids[pos // block_m + b] = e
        pos += nblk * block_m
    return np.array(sorted_ids, np.int32), np.array(expert_ids, np.int32), pos
