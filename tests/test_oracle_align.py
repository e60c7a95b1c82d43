"""Pins for the oracle's token-to-expert sort and padding (CPU only)."""
import numpy as np
import pytest

from conftest import load_golden
from oracle import align as A


def test_fixture_hand_worked():
    g = load_golden("moe_align_tiny.json")
    s, e, npp = A.moe_align(np.array(g["topk_ids"], np.int32), g["experts"], g["block_m"])
    assert s.tolist() == g["sorted_ids"]
    assert e.tolist() == g["expert_ids"]
    assert npp == g["num_post_pad"]
    s2, e2, npp2 = A.moe_align_bruteforce(np.array(g["topk_ids"], np.int32), g["experts"], g["block_m"])
    assert s2.tolist() == g["sorted_ids"] and e2.tolist() == g["expert_ids"] and npp2 == npp


@pytest.mark.parametrize("seed,t,topk,experts,bm", [(0, 7, 2, 5, 4), (1, 33, 3, 8, 16), (2, 1, 1, 4, 16),
                                                     (3, 50, 6, 64, 32), (4, 20, 4, 3, 1)])
def test_vectorised_equals_bruteforce(seed, t, topk, experts, bm):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, experts, size=(t, topk)).astype(np.int32)
    if t > 3:
        ids[0, 0] = -1
        ids[2, -1] = experts + 3      # invalid ids are dropped
    a = A.moe_align(ids, experts, bm)
    b = A.moe_align_bruteforce(ids, experts, bm)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and a[2] == b[2]


@pytest.mark.parametrize("skew", [False, True])
def test_invariants(skew):
    rng = np.random.default_rng(7)
    t, topk, experts, bm = 200, 6, 64, 16
    ids = np.stack([rng.permutation(experts)[:topk] for _ in range(t)]).astype(np.int32)
    if skew:
        ids[:, 0] = 0                 # one very hot expert
    s, e, npp = A.moe_align(ids, experts, bm)
    cap_sorted, cap_blocks = A.capacity(t, topk, experts, bm)
    assert s.size == cap_sorted and e.size == cap_blocks
    flat = ids.reshape(-1)
    real = s[:npp][s[:npp] != t * topk]
    assert sorted(real.tolist()) == list(range(t * topk))     # a permutation of all flat indices
    assert npp % bm == 0 and np.all(s[npp:] == t * topk) and np.all(e[npp // bm:] == -1)
    for b in range(npp // bm):
        blk = s[b * bm:(b + 1) * bm]
        blk = blk[blk != t * topk]
        assert np.all(flat[blk] == e[b])
        assert np.all(np.diff(blk) > 0)                          # stable: ascending within a block
    assert np.all(np.diff(e[:npp // bm]) >= 0)                   # experts in ascending order


def test_capacity_bounds_every_routing():
    for t, topk, experts, bm in [(1, 1, 128, 16), (16, 8, 128, 16), (4096, 8, 128, 256), (3, 2, 4, 2)]:
        cap, blocks = A.capacity(t, topk, experts, bm)
        # worst case: every used expert leaves bm-1 padding slots
        used = min(experts, t * topk)
        assert cap >= t * topk + used * (bm - 1) and cap % bm == 0 and blocks * bm == cap


# ---- grouped-contiguous and grouped-masked organizations ---------------------------------

@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("bm", [1, 4, 16, 128])
def test_grouped_maps_equal_direct_construction(seed, bm):
    rng = np.random.default_rng(seed)
    e = int(rng.integers(1, 9))
    cnt = rng.integers(0, 40, size=e)
    cnt[rng.integers(0, e)] = 0                               # an empty expert
    offs = np.concatenate([[0], np.cumsum(cnt)])
    for extra in (None, int(offs[-1]) + 7):                  # trailing rows of no expert
        got = A.grouped_map("contiguous", offs, e, bm, rows_total=extra)
        ref = A.grouped_map_direct("contiguous", offs, e, bm, rows_total=extra)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]) and got[2] == ref[2]
    cap = 32
    counts = rng.integers(-3, 40, size=e)                     # clamped to [0, cap]
    got = A.grouped_map("masked", counts, e, bm, cap)
    ref = A.grouped_map_direct("masked", counts, e, bm, cap)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1]) and got[2] == ref[2]


def test_grouped_map_invariants():
    offs = np.array([0, 5, 5, 12])
    s, eid, npp = A.grouped_map("contiguous", offs, 3, 4)
    assert npp == 8 + 8                                        # 5 -> 8, 0 -> 0, 7 -> 8
    assert list(s[:8]) == [0, 1, 2, 3, 4, 12, 12, 12] and list(s[8:16]) == [5, 6, 7, 8, 9, 10, 11, 12]
    assert list(eid[:4]) == [0, 0, 2, 2]
    s, eid, npp = A.grouped_map("masked", np.array([2, 0, 3]), 3, 2, cap=4)
    assert list(s[:npp]) == [0, 1, 8, 9, 10, 12] and list(eid[:3]) == [0, 2, 2]
