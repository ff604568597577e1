"""Pins of the oracle's segment reference (CPU only).

The grouping it follows: tokens grouped by adapter (Fastino article: the
kernel "groups a batch's tokens by adapter"), contiguous segments of tokens
sharing an adapter (study page, section "The kernel trick").  Readings: slots
ascending, original order inside a segment, -1 and out-of-range ids dropped.

Pinned against a brute force that scans slots one by one (a different
algorithm from the stable argsort) and against the invariants every valid
grouping has.
"""
import numpy as np
import pytest

from oracle import lora_oracle as lo


def brute(ids, n_slots):
    perm, starts, slots = [], [0], []
    for s in range(n_slots):
        members = [i for i, a in enumerate(ids) if a == s]
        if members:
            perm += members
            starts.append(len(perm))
            slots.append(s)
    bad = sum(1 for a in ids if a < -1 or a >= n_slots)
    return perm, starts, slots, bad


def check_invariants(ids, n_slots, seg):
    ids = np.asarray(ids)
    perm, ss, sl = seg["perm"], seg["seg_start"], seg["seg_slot"]
    active = np.nonzero((ids >= 0) & (ids < n_slots))[0]
    assert sorted(perm.tolist()) == active.tolist()           # a permutation of the active tokens
    assert np.all(np.diff(ids[perm]) >= 0)                     # ids non-decreasing along perm
    assert ss[0] == 0 and ss[-1] == len(perm) == seg["n_active"]
    assert len(sl) == seg["n_seg"] == len(np.unique(ids[active]))
    for k in range(seg["n_seg"]):
        part = perm[ss[k]:ss[k + 1]]
        assert len(part) > 0
        assert np.all(ids[part] == sl[k])
        assert np.all(np.diff(part) > 0)                       # original order inside a run
    assert seg["max_seg_len"] == (int(np.max(np.diff(ss))) if seg["n_seg"] else 0)


CASES = {
    "empty": ([], 4),
    "one": ([2], 4),
    "all_neg": ([-1] * 9, 3),
    "one_id": ([1] * 17, 3),
    "all_distinct": (list(range(31, -1, -1)), 32),
    "last_slot": ([7, 7, -1, 7], 8),
    "out_of_range": ([0, 5, -2, 1, 100, -1, 1], 4),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_edge_cases(name):
    ids, n_slots = CASES[name]
    seg = lo.build_segments(ids, n_slots)
    perm, starts, slots, bad = brute(ids, n_slots)
    assert seg["perm"].tolist() == perm
    assert seg["seg_start"].tolist() == starts
    assert seg["seg_slot"].tolist() == slots
    assert seg["n_bad"] == bad
    check_invariants(ids, n_slots, seg)


@pytest.mark.parametrize("seed", range(20))
def test_random_against_brute_force(seed):
    rng = np.random.default_rng(seed)
    n_slots = int(rng.integers(1, 40))
    n = int(rng.integers(0, 300))
    ids = rng.integers(-2, n_slots + 2, n).tolist()
    seg = lo.build_segments(ids, n_slots)
    perm, starts, slots, bad = brute(ids, n_slots)
    assert seg["perm"].tolist() == perm
    assert seg["seg_start"].tolist() == starts
    assert seg["seg_slot"].tolist() == slots
    assert seg["n_bad"] == bad
    check_invariants(ids, n_slots, seg)


def test_planted_unstable_order_is_caught(monkeypatch):
    """A grouping that reverses order inside a segment fails the brute-force pin."""
    real = lo.build_segments

    def reversed_runs(ids, n_slots):
        seg = real(ids, n_slots)
        p = seg["perm"].copy()
        for k in range(seg["n_seg"]):
            a, b = seg["seg_start"][k], seg["seg_start"][k + 1]
            p[a:b] = p[a:b][::-1]
        seg["perm"] = p
        return seg

    monkeypatch.setattr(lo, "build_segments", reversed_runs)
    ids = [1, 0, 1, 1, 0]
    assert lo.build_segments(ids, 2)["perm"].tolist() != brute(ids, 2)[0]
