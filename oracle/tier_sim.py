"""Two-tier adapter cache: the reference policy.  TEST INFRASTRUCTURE ONLY
(the same rules as ``lora_oracle``: only tests, the smoke check and the CPU
baseline of the benchmark use it; the library shares no code with it).

Study page "Multi-LoRA Serving - S-LoRA/Punica Batching, Adapter Hot-Swap &
Memory", section "Memory: slots, tiers and paging" and its cache simulation:
adapters live in GPU slots (few, fast), behind them a larger host-memory LRU
(a swap is a PCIe copy), behind that a cold store.  For each request:

* the GPU tier is consulted first, in least-recently-used order: a hit
  refreshes the adapter; a miss brings the adapter into the GPU tier and, if
  the tier is over capacity, drops its least recently used adapter;
* only on a GPU miss is the host tier consulted, with the same LRU rule: a
  hit is a host-to-GPU copy, a miss is a load from the cold store.

The expected load wait per request weighs host hits by the host copy time
and cold loads by the cold load time (the page's example: 3 ms and 120 ms).

Slot numbers (not in the page's simulation, needed to drive a slot pool): an
adapter entering the GPU tier takes the lowest free slot, else the slot of
the adapter it displaces.
"""
from __future__ import annotations

from collections import OrderedDict
from typing import Dict, List, Sequence

GPU_HIT, HOST_HIT, COLD = 0, 1, 2


class LRUTier:
    """Least-recently-used set of adapter ids with a capacity."""

    def __init__(self, capacity: int):
        self.capacity = capacity
        self.order: "OrderedDict[int, None]" = OrderedDict()   # least recent first

    def access(self, key: int):
        """Returns (hit, evicted key or None).  A miss inserts the key as the
        most recent; past capacity the least recent key leaves."""
        if key in self.order:
            self.order.move_to_end(key)
            return True, None
        self.order[key] = None
        evicted = None
        if len(self.order) > self.capacity:
            evicted, _ = self.order.popitem(last=False)
        return False, evicted


def simulate(trace: Sequence[int], gpu_slots: int, host_slots: int) -> Dict[str, List[int]]:
    """Per request: tier it was served from, its GPU slot afterwards (-1 if
    it left again at once, possible only with capacity 0), and the adapter it
    displaced from the GPU tier (-1 none)."""
    gpu, host = LRUTier(gpu_slots), LRUTier(host_slots)
    slot_of: Dict[int, int] = {}
    free = list(range(gpu_slots))   # lowest first
    tiers, slots, evicted = [], [], []
    for a in trace:
        a = int(a)
        hit, out = gpu.access(a)
        if hit:
            tiers.append(GPU_HIT)
        else:
            if out is not None and out != a:
                s = slot_of.pop(out)
            else:
                s = free.pop(0) if free else -1
            if out != a:
                slot_of[a] = s
            h_hit, _ = host.access(a)
            tiers.append(HOST_HIT if h_hit else COLD)
        slots.append(slot_of.get(a, -1))
        evicted.append(-1 if hit or out is None else out)
    return {"tier": tiers, "slot": slots, "evicted": evicted}


def table_row(tiers: Sequence[int], host_ms: float, cold_ms: float) -> Dict[str, float]:
    """Share of requests served from the GPU and from the host (percent), the
    number of cold loads, and the mean load wait per request (ms)."""
    n = len(tiers)
    g = sum(1 for t in tiers if t == GPU_HIT)
    h = sum(1 for t in tiers if t == HOST_HIT)
    c = n - g - h
    return {"gpu_pct": 100.0 * g / n, "host_pct": 100.0 * h / n, "cold_loads": c,
            "mean_wait_ms": (h * host_ms + c * cold_ms) / n}
