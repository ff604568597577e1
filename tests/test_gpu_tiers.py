"""GPU: lora_tiers_acquire serving consecutive decode batches from a pool with
fewer slots than adapters.  Each batch's adapter ids go through the tiers,
which evict and upload adapters (asynchronously, from page-locked host
buffers) on the stream; the batch is then applied with the slot ids the
acquire returned.  Checked against the fp64 oracle, which knows only the
adapter ids, and against the policy oracle's counts."""
import numpy as np
import pytest

import workloads as W
from oracle import lora_oracle as lo
from oracle import tier_sim as T

from gpu_util import assert_close, say

pytestmark = pytest.mark.gpu


def test_acquire_serves_batches_through_four_slots():
    import torch
    import segmented_gathered_rank_amd as sgr
    from segmented_gathered_rank_amd.harness import from_device, to_device
    wl = W.tier_batches()
    bsz = wl.notes["batch"]
    mod = wl.modules[0]
    n_slots, host_slots = 4, 6
    say(f"tiers: {wl.n_slots} adapters, {n_slots} GPU slots, host tier {host_slots}, "
        f"{wl.n_tokens // bsz} batches of {bsz}")
    pages = n_slots * 16 * (mod.h_in + mod.h_out) // wl.page_elems
    pool = sgr.lora_pool_create(0, sgr.LORA_BF16, wl.page_elems, pages, n_slots, 1, [mod.h_in], [mod.h_out], 16)
    tiers = sgr.lora_tiers_create(n_slots, host_slots)
    fetched = []

    def fetch(adapter, module):
        fetched.append(adapter)
        a = wl.adapters[adapter][module]
        return None if a is None else (a[0], a[1], a[2], a[3])

    dev = torch.device("cuda", 0)
    x = to_device(wl.x[0], "bf16", dev)
    y = to_device(wl.y0[0], "bf16", dev)
    nb = sgr.lora_segments_bytes(bsz, n_slots)
    seg_buf = torch.zeros(max(nb, 256), dtype=torch.uint8, device=dev)
    seg = sgr.lora_segments_bind(seg_buf, bsz, n_slots)
    requests = []
    for b in range(wl.n_tokens // bsz):
        ids = wl.ids[b * bsz:(b + 1) * bsz]
        req = ids[ids >= 0]
        slots = sgr.lora_tiers_acquire(tiers, pool, req, fetch)
        requests.extend(req.tolist())
        tok_slots = np.full(bsz, -1, np.int32)
        tok_slots[ids >= 0] = slots
        for a, s in zip(req.tolist(), slots.tolist()):   # one slot per adapter within a batch
            assert sgr.lora_tiers_slot_of(tiers, a) == s
        d_ids = torch.from_numpy(tok_slots).to(dev)
        sgr.lora_build_segments(d_ids, seg)
        sgr.lora_apply_bgmv(pool, 0, 1, x[b * bsz:], mod.h_in, 0, seg, y[b * bsz:], mod.h_out, 0, sgr.LORA_BF16)
    torch.cuda.synchronize()
    got = lo.decode(from_device(y), "bf16")
    ref = lo.apply_to_y0(wl, 0)
    assert_close(got, ref, "bf16", "tiers")
    # the engine's counts are the policy oracle's on the same request sequence
    sim = T.simulate(requests, n_slots, host_slots)
    st = sgr.lora_tiers_stats(tiers)
    assert st["gpu_hits"] == sum(t == T.GPU_HIT for t in sim["tier"])
    assert st["host_hits"] == sum(t == T.HOST_HIT for t in sim["tier"])
    assert st["cold_loads"] == sum(t == T.COLD for t in sim["tier"]) == len(fetched)
    assert st["host_hits"] > 0 and st["cold_loads"] > n_slots   # both paths were exercised
    ps = sgr.lora_pool_stats(pool)
    assert ps["loaded_slots"] <= n_slots and ps["evicts"] > 0
    sgr.lora_tiers_destroy(tiers)
    sgr.lora_pool_destroy(pool)


def test_acquire_errors():
    import segmented_gathered_rank_amd as sgr
    wl = W.tier_batches(seed=22)
    mod = wl.modules[0]
    pool = sgr.lora_pool_create(0, sgr.LORA_BF16, wl.page_elems, 4 * 16 * 10, 4, 1, [mod.h_in], [mod.h_out], 16)
    fetch = lambda a, m: (wl.adapters[a][m][0], wl.adapters[a][m][1], wl.adapters[a][m][2], wl.adapters[a][m][3])
    tiers = sgr.lora_tiers_create(4, 6)
    with pytest.raises(sgr.LoraError) as ei:           # five adapters for four slots
        sgr.lora_tiers_acquire(tiers, pool, [0, 1, 2, 3, 4], fetch)
    assert ei.value.status == -5
    assert sgr.lora_tiers_stats(tiers) == {"gpu_hits": 0, "host_hits": 0, "cold_loads": 0}   # nothing touched

    def bad(a, m):
        raise RuntimeError("cold store unavailable")
    with pytest.raises(RuntimeError):
        sgr.lora_tiers_acquire(tiers, pool, [5], bad)
    sgr.lora_tiers_destroy(tiers)
    no_host = sgr.lora_tiers_create(4, 0)                # uploads need a host tier
    with pytest.raises(sgr.LoraError) as ei:
        sgr.lora_tiers_acquire(no_host, pool, [1], fetch)
    assert ei.value.status == -1
    sgr.lora_tiers_destroy(no_host)
    sgr.lora_pool_destroy(pool)


def test_prefetch_on_a_copy_stream():
    """The next batch's adapters are uploaded on a second stream while the
    current batch computes (the slide-9 forecast, here the exact next batch).
    Every batch still matches the oracle, and more requests find their adapter
    on the GPU than without the forecast."""
    import torch
    import segmented_gathered_rank_amd as sgr
    from segmented_gathered_rank_amd.harness import from_device, to_device
    wl = W.tier_batches(seed=23, n_batches=12)
    bsz = wl.notes["batch"]
    mod = wl.modules[0]
    n_slots, host_slots = 8, 6
    say(f"prefetch: {wl.n_slots} adapters, {n_slots} GPU slots, host tier {host_slots}")
    pages = n_slots * 16 * (mod.h_in + mod.h_out) // wl.page_elems
    pool = sgr.lora_pool_create(0, sgr.LORA_BF16, wl.page_elems, pages, n_slots, 1, [mod.h_in], [mod.h_out], 16)
    tiers = sgr.lora_tiers_create(n_slots, host_slots)

    def fetch(adapter, module):
        a = wl.adapters[adapter][module]
        return None if a is None else (a[0], a[1], a[2], a[3])

    dev = torch.device("cuda", 0)
    compute = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    x = to_device(wl.x[0], "bf16", dev)
    y = to_device(wl.y0[0], "bf16", dev)
    seg_buf = torch.zeros(max(sgr.lora_segments_bytes(bsz, n_slots), 256), dtype=torch.uint8, device=dev)
    seg = sgr.lora_segments_bind(seg_buf, bsz, n_slots)
    nb = wl.n_tokens // bsz
    reqs = [wl.ids[b * bsz:(b + 1) * bsz][wl.ids[b * bsz:(b + 1) * bsz] >= 0] for b in range(nb)]
    issued = 0
    for b in range(nb):
        ids = wl.ids[b * bsz:(b + 1) * bsz]
        slots = sgr.lora_tiers_acquire(tiers, pool, reqs[b], fetch, compute)
        tok_slots = np.full(bsz, -1, np.int32)
        tok_slots[ids >= 0] = slots
        d_ids = torch.from_numpy(tok_slots).to(dev)
        sgr.lora_build_segments(d_ids, seg, compute)
        sgr.lora_apply_bgmv(pool, 0, 1, x[b * bsz:], mod.h_in, 0, seg, y[b * bsz:], mod.h_out, 0, sgr.LORA_BF16,
                            compute)
        sgr.lora_tiers_batch_done(tiers, compute)
        if b + 1 < nb:
            issued += sgr.lora_tiers_prefetch(tiers, pool, reqs[b + 1], fetch, copy)
    torch.cuda.synchronize()
    got = lo.decode(from_device(y), "bf16")
    assert_close(got, lo.apply_to_y0(wl, 0), "bf16", "tiers with prefetch")
    st = sgr.lora_tiers_stats(tiers)
    plain = T.simulate([int(a) for r in reqs for a in r], n_slots, host_slots)
    plain_hits = sum(t == T.GPU_HIT for t in plain["tier"])
    say(f"  GPU hits {st['gpu_hits']} with the forecast ({issued} uploads issued), {plain_hits} without")
    assert issued > 0 and st["gpu_hits"] > plain_hits
    sgr.lora_tiers_destroy(tiers)
    sgr.lora_pool_destroy(pool)
