"""Pins for the oracle's route pack (CPU only): brute-force sorting, the
route fixtures the pages print, and the table invariants."""
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def brute_pack(ids, E):
    M, k = ids.shape
    flat = ids.ravel()
    valid = [s for s in range(M * k) if 0 <= flat[s] < E]
    order = sorted(valid, key=lambda s: (flat[s], s))
    offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + sum(1 for s in valid if flat[s] == e)
    t2p = [-1] * (M * k)
    for pos, s in enumerate(order):
        t2p[s] = pos
    active = sorted(set(int(flat[s]) for s in valid))
    invalid = sum(1 for s in range(M * k) if not (0 <= flat[s] < E) and flat[s] != -1)
    return dict(expert_offsets=np.array(offsets), sorted_slot=np.array(order, dtype=np.int64),
                sorted_token=np.array([s // k for s in order], dtype=np.int64),
                token_to_perm=np.array(t2p), active_experts=np.array(active, dtype=np.int64),
                num_active=len(active), invalid=invalid)


def check_same(got, ref):
    for key in ("expert_offsets", "sorted_slot", "sorted_token", "token_to_perm", "active_experts"):
        assert np.array_equal(np.asarray(got[key], np.int64), np.asarray(ref[key], np.int64)), key
    assert got["num_active"] == ref["num_active"]
    assert got["invalid"] == ref["invalid"]


def invariants(got, ids, E):
    off = got["expert_offsets"]
    assert off[0] == 0 and np.all(np.diff(off) >= 0)
    nv = int(((ids >= 0) & (ids < E)).sum())
    assert off[E] == nv
    ss, t2p = got["sorted_slot"], got["token_to_perm"]
    for pos, s in enumerate(ss):
        assert t2p[s] == pos
        e = ids.flat[s]
        assert off[e] <= pos < off[e + 1]


def owner_spread_routes(tokens, experts, slots_per_rank, token_step, slot_step, offset):
    """Routes of the page's dynamic owner fixture ("memra-engine 0.108.0 --
    src/bin/ep_step_fp8_gate.rs", benchmark_tests, fn
    dynamic_grouped_selected_routes), built from its description: the experts
    split into len(slots_per_rank) equal contiguous ranges, the top-k slots
    handed to the ranges in order, slots_per_rank[r] of them to range r, and
    slot j of token t taking the expert at local index
    (token_step*t + slot_step*j + offset) mod the range size."""
    ranks = len(slots_per_rank)
    per = experts // ranks
    rank_of_slot = np.repeat(np.arange(ranks), slots_per_rank)
    t = np.arange(tokens)[:, None]
    j = np.arange(rank_of_slot.size)[None, :]
    return (rank_of_slot[None, :] * per + (token_step * t + slot_step * j + offset) % per).astype(np.int32)


def _golden():
    d = {}
    for line in open(os.path.join(GOLDEN, "route_fixtures.txt")):
        if line.strip() and not line.startswith("#"):
            p = line.split()
            d[p[0]] = [int(v) for v in p[1:]]
    return d


def test_page_route_fixtures_and_their_packs():
    g = _golden()
    # the page prints both rows of its two-token fixture: they are the input
    r = np.array([g["grouped_2_288_token0"], g["grouped_2_288_token1"]], np.int32)
    got = oracle.route_pack(r, 288)
    check_same(got, brute_pack(r, 288))
    # expert j*36 holds slot j (token 0) and expert j*36+1 holds slot 8+j
    assert list(got["active_experts"]) == sorted(g["grouped_2_288_token0"] + g["grouped_2_288_token1"])
    # four ranks of 72 experts; slots 0 | 1-2 | 3-5 | 6-7 per rank
    d = owner_spread_routes(3, 288, [1, 2, 3, 2], token_step=11, slot_step=7, offset=1)
    assert all(len(set(row)) == 8 for row in d.tolist())     # no duplicate route in a token
    counts = np.bincount(d.ravel() // 72, minlength=4)
    assert list(counts) == g["dynamic_3_288_4_owner_counts"]
    got = oracle.route_pack(d, 288)
    check_same(got, brute_pack(d, 288))
    # per-owner slot counts are the prefix-offset differences at owner borders
    off = got["expert_offsets"]
    assert [off[72 * (o + 1)] - off[72 * o] for o in range(4)] == g["dynamic_3_288_4_owner_counts"]


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_pack_matches_brute_force_on_every_workload(name):
    wl = workloads.WORKLOADS[name]
    M = min(wl.M, 256)  # brute force is quadratic; the GPU tests cover full M
    ids, _, _ = workloads.make_routes(wl, 0, M=M)
    got = oracle.route_pack(ids, wl.experts)
    check_same(got, brute_pack(ids, wl.experts))
    invariants(got, ids, wl.experts)


@pytest.mark.parametrize("case", ["one_expert", "E1", "k_eq_E", "invalid", "all_invalid", "dups"])
def test_pack_adversarial(case):
    rng = np.random.default_rng(3)
    if case == "one_expert":
        ids, E = np.full((37, 4), 5, np.int32), 9
    elif case == "E1":
        ids, E = np.zeros((13, 1), np.int32), 1
    elif case == "k_eq_E":
        E = 6
        ids = np.stack([rng.permutation(E) for _ in range(11)]).astype(np.int32)
    elif case == "invalid":
        E = 8
        ids = rng.integers(0, E, (20, 3)).astype(np.int32)
        ids[2, 1], ids[5, 0], ids[7, 2], ids[9, 1] = -1, E, -7, 1 << 30
    elif case == "all_invalid":
        E = 4
        ids = np.full((3, 2), -1, np.int32)
        ids[1, 1] = 99
    else:
        E = 5
        ids = rng.integers(0, E, (9, 4)).astype(np.int32)
    got = oracle.route_pack(ids, E)
    ref = brute_pack(ids, E)
    check_same(got, ref)
    invariants(got, ids, E)
