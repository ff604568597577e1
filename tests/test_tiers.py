"""Adapter tiers (GPU slots <- host memory <- cold store): the oracle policy
pinned to the study page's printed cache simulation and to hand-derived
cases, then the library's native engine checked against the oracle request
by request.  CPU only: the engine is host code."""
import json
import os

import numpy as np
import pytest

import workloads as W
from oracle import tier_sim as T

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cache_simulation.json")


def test_oracle_reproduces_the_pages_table():
    g = json.load(open(GOLDEN))
    s = g["setting"]
    trace = W.request_trace(s["lcg_seed"], s["adapters"], s["requests"], s["zipf_s"])
    for row in g["rows"]:
        r = T.table_row(T.simulate(trace, row["gpu_slots"], row["host_slots"])["tier"],
                        s["host_copy_ms"], s["cold_load_ms"])
        assert f"{r['gpu_pct']:.1f}" == row["gpu_hit_pct"], row
        assert f"{r['host_pct']:.1f}" == row["host_hit_pct"], row
        assert r["cold_loads"] == row["cold_loads"], row
        assert f"{r['mean_wait_ms']:.2f}" == row["mean_wait_ms"], row


def test_lcg_first_draws():
    # the recurrence by hand from seed 11: 11*1664525 + 1013904223 = 1032213998
    s1 = 1032213998
    s2 = (s1 * 1664525 + 1013904223) % 2 ** 32
    u = W.lcg_uniforms(11, 2)
    assert u[0] == s1 / 2 ** 32 and u[1] == s2 / 2 ** 32


def test_policy_by_hand():
    """GPU tier 2, host tier 2, requests 1 2 1 3 2:
    1 cold -> slot 0; 2 cold -> slot 1; 1 GPU hit; 3 misses, displaces the
    least recent (2) and takes slot 1, host tier {1,2} drops 1 for 3, cold;
    2 misses, displaces 1 (slot 0), host tier {2,3} has 2: host hit."""
    out = T.simulate([1, 2, 1, 3, 2], 2, 2)
    assert out["tier"] == [T.COLD, T.COLD, T.GPU_HIT, T.COLD, T.HOST_HIT]
    assert out["slot"] == [0, 1, 0, 1, 0]
    assert out["evicted"] == [-1, -1, -1, 2, 1]


def test_policy_invariants():
    rng = np.random.default_rng(3)
    # no more distinct adapters than GPU slots: only first touches miss, all cold
    tr = rng.integers(0, 6, size=300)
    out = T.simulate(tr, 6, 0)
    assert sum(t != T.GPU_HIT for t in out["tier"]) == len(set(tr.tolist()))
    # cycling over one more adapter than slots defeats LRU: every request misses
    tr = np.tile(np.arange(5), 20)
    out = T.simulate(tr, 4, 10)
    assert all(t != T.GPU_HIT for t in out["tier"])
    assert out["tier"][5:] == [T.HOST_HIT] * (len(tr) - 5)
    # no host tier: every GPU miss is a cold load; slots stay in range
    tr = rng.integers(0, 40, size=500)
    out = T.simulate(tr, 8, 0)
    assert all(t in (T.GPU_HIT, T.COLD) for t in out["tier"])
    assert all(0 <= s < 8 for s in out["slot"])


def _engine(gpu, host, trace):
    import segmented_gathered_rank_amd as sgr
    t = sgr.lora_tiers_create(gpu, host)
    try:
        tier, slot, ev = sgr.lora_tiers_touch(t, trace)
        stats = sgr.lora_tiers_stats(t)
    finally:
        sgr.lora_tiers_destroy(t)
    return tier, slot, ev, stats


def test_engine_matches_oracle_on_the_pages_trace():
    trace = W.request_trace()
    for gpu, host in [(8, 100), (32, 100), (32, 500), (128, 500)]:
        tier, slot, ev, stats = _engine(gpu, host, trace)
        ref = T.simulate(trace, gpu, host)
        assert np.array_equal(tier, ref["tier"]) and np.array_equal(slot, ref["slot"])
        assert np.array_equal(ev, ref["evicted"])
        assert stats["cold_loads"] == sum(t == T.COLD for t in ref["tier"])


@pytest.mark.parametrize("gpu,host,n_ids,seed", [(1, 0, 5, 1), (1, 3, 4, 2), (3, 1, 9, 3), (5, 5, 5, 4),
                                                  (16, 64, 300, 5), (64, 8, 100, 6)])
def test_engine_matches_oracle_on_random_traces(gpu, host, n_ids, seed):
    rng = np.random.default_rng(seed)
    trace = rng.integers(0, n_ids, size=2000).astype(np.int32)
    tier, slot, ev, _ = _engine(gpu, host, trace)
    ref = T.simulate(trace, gpu, host)
    assert np.array_equal(tier, ref["tier"]) and np.array_equal(slot, ref["slot"])
    assert np.array_equal(ev, ref["evicted"])


def test_engine_arguments():
    import segmented_gathered_rank_amd as sgr
    with pytest.raises(sgr.LoraError):
        sgr.lora_tiers_create(0, 4)
    with pytest.raises(sgr.LoraError):
        sgr.lora_tiers_create(4, -1)
    t = sgr.lora_tiers_create(4, 4)
    with pytest.raises(sgr.LoraError):
        sgr.lora_tiers_touch(t, [1, -2])
    assert sgr.lora_tiers_slot_of(t, 7) == -1
    sgr.lora_tiers_touch(t, [7])
    assert sgr.lora_tiers_slot_of(t, 7) == 0
    sgr.lora_tiers_destroy(t)
