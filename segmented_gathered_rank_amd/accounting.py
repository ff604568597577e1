"""Algorithmic work of a multi-LoRA apply step (bytes and FLOPs), for rooflines.

Only what the method has to move or compute is counted:
  * x read once per distinct input (modules that share x count it once),
  * y read and written once for every token that has an adapter,
  * each distinct adapter's A and B pages read once per batch and module,
  * t written and read back once on the two-kernel (shrink, expand) path,
  * ids read and the token permutation written by the segment build.
Re-reads that the method avoids (per-token reads of A and B) are not counted.

FLOPs per token and module: 2 * rank * (h_in + h_out) (the shrink and the
expand).  Against the base product's 2 * h_in * h_out this is the study page's
"about 2r/d extra FLOPs per adapted layer" (section "Strategies compared";
its demo prints 1.56% for d = 2048, r = 16).
"""
from __future__ import annotations

from typing import Dict

import numpy as np


def flop_overhead_ratio(rank: int, d: int) -> float:
    """Adapter FLOPs over base FLOPs for one square d x d layer: 2*r*d*2 / (2*d*d)."""
    return (2 * rank * d * 2) / (2 * d * d)


def adapter_bytes(rank: int, h_in: int, h_out: int, elem_bytes: int) -> int:
    """Bytes of one adapter (A and B) for one layer."""
    return rank * (h_in + h_out) * elem_bytes


def base_layer_bytes(h_in: int, h_out: int, elem_bytes: int) -> int:
    return h_in * h_out * elem_bytes


def step_work(wl, fused: bool, y_elem_bytes: int = None) -> Dict[str, object]:
    """Algorithmic bytes and FLOPs of one step over all modules of ``wl``.

    fused=True: one-launch BGMV (t stays on chip).  fused=False: shrink then
    expand with t through memory.  Returns totals and per-module figures.
    """
    eb = 2 if wl.dtype == "bf16" else 4
    yb = y_elem_bytes or eb
    ids = np.asarray(wl.ids)
    seen_x = set()
    per_module = []
    tot_b = tot_f = 0
    for m, mod in enumerate(wl.modules):
        rank_of = {}
        for s in np.unique(ids):
            if 0 <= s < wl.n_slots and wl.adapters[s][m] is not None:
                rank_of[int(s)] = int(wl.adapters[s][m][0])
        active = np.array([int(i) in rank_of for i in ids]) if ids.size else np.zeros(0, bool)
        n_act = int(active.sum())
        xb = 0
        if mod.x_group not in seen_x:
            xb = n_act * mod.h_in * eb
            seen_x.add(mod.x_group)
        ab = sum(adapter_bytes(r, mod.h_in, mod.h_out, eb) for r in rank_of.values())
        ybytes = 2 * n_act * mod.h_out * yb
        ranks = np.array([rank_of.get(int(i), 0) for i in ids])
        tb = 0 if fused else 2 * int(ranks.sum()) * 4
        flops = int(2 * ranks.sum() * (mod.h_in + mod.h_out))
        b = xb + ab + ybytes + tb
        per_module.append({"bytes": b, "flops": flops, "x": xb, "adapters": ab, "y": ybytes, "t": tb})
        tot_b += b
        tot_f += flops
    seg_bytes = 4 * ids.size * 2
    return {"bytes": tot_b, "flops": tot_f, "segment_bytes": seg_bytes, "per_module": per_module}
