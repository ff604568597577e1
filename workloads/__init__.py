"""Seeded synthetic inputs for the multi-LoRA apply path.

This module is shared by the CPU oracle (under ``oracle/``) and by the GPU
path's tests and benchmark.  It holds no arithmetic of the method itself: it
only draws random numbers, rounds them to the storage dtype and lays out the
structure of each workload (adapter ids, segment lengths, ranks, scales).

Layout of every workload (row-major, little endian):

* ``x[g]``   [n_tokens, h_in]   input rows; module ``m`` reads ``x[module.x_group]``
* ``W[m]``   [h_in, h_out]      shared base weight of module ``m``
* ``A``      [rank, h_in]       one adapter's down-projection, one row per rank row
* ``B``      [rank, h_out]      one adapter's up-projection, one row per rank row
* ``y0[m]``  [n_tokens, h_out]  the buffer the library adds the adapter term into
* ``ids``    [n_tokens] int32   adapter slot per token, -1 = no adapter

With this layout the adapted linear layer of the "Multi-LoRA Serving" study
page (section "The kernel trick: gather, do not merge") reads
``y_i = x_i W + scale_a * (x_i A_a^T) B_a``; its ``A_a`` is our ``A`` and its
``B_a`` is our ``B`` transposed.

Storage: dtype ``"f32"`` arrays are ``numpy.float32``; dtype ``"bf16"`` arrays
are ``numpy.uint16`` holding bfloat16 bit patterns, rounded from float32 draws
to nearest-even.  Each side decodes those bits with its own code.

Seeds: workload ``Cc`` uses ``numpy.random.default_rng(c)``; draws happen in the
order structure -> ids -> x -> W -> A -> B -> y0.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Module", "Workload", "to_bf16_bits", "zipf_ids", "finite_zipf_cdf",
    "c0_worked_example", "c1_tiny_f32", "c2_bgmv_decode", "c3_sgmv_prefill",
    "c4_mixed_rank", "c5_encoder_step", "fused_tiles", "fingerprint_rank1", "integer_exact",
    "lcg_uniforms", "request_trace", "tier_batches", "with_fp8_base", "fp8_code_sweep",
    "BY_NAME",
]


# --------------------------------------------------------------------------
# storage helpers
# --------------------------------------------------------------------------
def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); return the bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.uint16)
    flat_in, flat_out = a.reshape(-1), out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        u = flat_in[s:s + step].view(np.uint32).copy()
        u += np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
        u >>= np.uint32(16)
        flat_out[s:s + step] = u
    return out


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    if dtype == "bf16":
        return to_bf16_bits(a32)
    raise ValueError(dtype)


def finite_zipf_cdf(n: int, s: float) -> np.ndarray:
    """Cumulative weights of the finite Zipf law over ranks 1..n (weight 1/k^s).

    Same construction as the cache simulation of the "Multi-LoRA Serving"
    study page (section "Memory: slots, tiers and paging", its sampler): weights
    1/(i+1)^s, normalised running sum.
    """
    w = 1.0 / np.power(np.arange(1, n + 1, dtype=np.float64), s)
    return np.cumsum(w / w.sum())


def zipf_ids(rng: np.random.Generator, count: int, n: int, s: float) -> np.ndarray:
    """Draw ``count`` slots from a finite Zipf(s) over n slots, slot 0 hottest.

    Inverse-CDF sampling: u ~ U[0,1), first index whose cdf >= u (a binary
    search, as the study page's sampler does)."""
    cdf = finite_zipf_cdf(n, s)
    u = rng.random(count)
    return np.minimum(np.searchsorted(cdf, u, side="left"), n - 1).astype(np.int32)


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------
@dataclasses.dataclass
class Module:
    name: str
    h_in: int
    h_out: int
    x_group: int          # index into Workload.x


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                       # "f32" or "bf16": storage of x, W, A, B, y0
    page_elems: int                  # elements per page of the paged adapter store
    n_slots: int
    modules: List[Module]
    ids: np.ndarray                  # int32 [n_tokens]
    x: List[np.ndarray]              # per x-group, [n_tokens, h_in]
    y0: List[np.ndarray]             # per module, [n_tokens, h_out]
    W: List[Optional[np.ndarray]]    # per module, [h_in, h_out] (None if not drawn)
    # adapters[slot][module] = (rank, scale, A [rank, h_in], B [rank, h_out]) or None
    adapters: List[List[Optional[Tuple[int, float, np.ndarray, np.ndarray]]]]
    notes: Dict[str, object] = dataclasses.field(default_factory=dict)
    # FP8 base (optional): per module, W as OCP E4M3 codes [h_in, h_out] (uint8)
    # and one float32 scale per output column [h_out]
    W8: Optional[List[Optional[np.ndarray]]] = None
    W8_scale: Optional[List[Optional[np.ndarray]]] = None

    @property
    def n_tokens(self) -> int:
        return int(self.ids.shape[0])

    @property
    def n_modules(self) -> int:
        return len(self.modules)

    def max_rank(self) -> int:
        r = [a[0] for row in self.adapters for a in row if a is not None]
        return max(r) if r else 1

    def pages_needed(self) -> int:
        h = self.page_elems
        tot = 0
        for row in self.adapters:
            for m, a in enumerate(row):
                if a is not None:
                    mod = self.modules[m]
                    tot += a[0] * (mod.h_in // h + mod.h_out // h)
        return tot


def _normal(rng, std, shape):
    """N(0, std) in float32 (std is the standard deviation)."""
    z = rng.standard_normal(shape, dtype=np.float32)
    z *= np.float32(std)
    return z


def _draw_values(rng, dtype, n_tokens, modules, x_groups, slot_ranks, scales,
                 x_std, w_std, ab_std, draw_w=True):
    """Draws x -> W -> A -> B -> y0 in that order (structure and ids come first)."""
    xs = []
    for g in range(x_groups):
        h_in = next(m.h_in for m in modules if m.x_group == g)
        xs.append(_store(_normal(rng, x_std, (n_tokens, h_in)), dtype))
    Ws = []
    for m in modules:
        Ws.append(_store(_normal(rng, w_std, (m.h_in, m.h_out)), dtype) if draw_w else None)
    adapters = []
    for s, ranks in enumerate(slot_ranks):
        row = []
        for mi, m in enumerate(modules):
            r = ranks[mi]
            A = _store(_normal(rng, ab_std, (r, m.h_in)), dtype)
            row.append([r, float(scales[s]), A, None])
        adapters.append(row)
    for s, row in enumerate(adapters):
        for mi, m in enumerate(modules):
            r = row[mi][0]
            row[mi][3] = _store(_normal(rng, ab_std, (r, m.h_out)), dtype)
            row[mi] = tuple(row[mi])
    y0 = []
    for m in modules:
        # stands in for the base product x.W: iid with the spread x.W would have
        y_std = x_std * w_std * np.sqrt(m.h_in)
        y0.append(_store(_normal(rng, y_std, (n_tokens, m.h_out)), dtype))
    return xs, Ws, adapters, y0


# --------------------------------------------------------------------------
# C0: the study page's worked example (fp32, d=2048, r=16, 50 adapters, batch 64)
# --------------------------------------------------------------------------
def c0_worked_example() -> Workload:
    """The numpy demo of the study page ("The kernel trick: gather, do not merge").

    fp32, d = 2048, rank 16, 50 adapters, 64 tokens, scale 2.  The draws keep the
    demo's seed and order (base weight, adapter down and up factors, activations,
    then the ids), which is what makes the page's count of 34 distinct adapters
    in the batch a usable check.  The page keeps W as [out][in], A as [adapter]
    [rank][in] and B as [adapter][out][rank]; this library's layout is their
    transpose for W and B (A rows are already rank rows).
    """
    d, r, n_ad, batch, scale = 2048, 16, 50, 64, 2.0
    draws = (("W", 0.02, (d, d)), ("A", 0.02, (n_ad, r, d)), ("B", 0.02, (n_ad, d, r)), ("X", 1.0, (batch, d)))
    rng = np.random.default_rng(0)
    page = {name: rng.normal(0, sigma, shape).astype(np.float32) for name, sigma, shape in draws}
    ids = rng.integers(0, n_ad, batch).astype(np.int32)
    A, B = page["A"], page["B"]
    adapters = [[(r, scale, np.ascontiguousarray(A[a]), np.ascontiguousarray(B[a].T))] for a in range(n_ad)]
    return Workload(
        name="c0_worked_example", dtype="f32", page_elems=d, n_slots=n_ad,
        modules=[Module("proj", d, d, 0)], ids=ids, x=[page["X"]], y0=[np.zeros((batch, d), np.float32)],
        W=[np.ascontiguousarray(page["W"].T)], adapters=adapters,
        notes={"W_page": page["W"], "A_page": A, "B_page": B})


# --------------------------------------------------------------------------
# C1: tiny fp32 SGMV
# --------------------------------------------------------------------------
def c1_tiny_f32(seed: int = 1) -> Workload:
    """h=64, 4 slots of rank 4, 16 tokens in 4 contiguous segments, one of them id -1.

    Segment lengths come from 3 distinct cut points in 1..15; the -1 segment sits
    at a uniform position; the other three take 3 distinct slots of the 4.
    x ~ N(0,1); W, A, B ~ N(0, 0.1); scale 2.0; fp32."""
    rng = np.random.default_rng(seed)
    h, n, n_slots, rank = 64, 16, 4, 4
    cuts = np.sort(rng.choice(np.arange(1, 16), 3, replace=False))
    bounds = np.concatenate([[0], cuts, [n]])
    neg_pos = int(rng.integers(0, 4))
    chosen = rng.choice(4, 3, replace=False)
    seg_ids, it = [], iter(chosen.tolist())
    for s in range(4):
        seg_ids.append(-1 if s == neg_pos else next(it))
    ids = np.empty(n, np.int32)
    for s in range(4):
        ids[bounds[s]:bounds[s + 1]] = seg_ids[s]
    mods = [Module("proj", h, h, 0)]
    xs, Ws, ad, y0 = _draw_values(rng, "f32", n, mods, 1, [[rank]] * n_slots,
                                  [2.0] * n_slots, 1.0, 0.1, 0.1)
    return Workload("c1_tiny_f32", "f32", 64, n_slots, mods, ids, xs, y0, Ws, ad,
                    notes={"segment_bounds": bounds, "segment_ids": seg_ids})


# --------------------------------------------------------------------------
# C2: BGMV decode
# --------------------------------------------------------------------------
def c2_bgmv_decode(seed: int = 2, n_modules: int = 1, n_tokens: int = 64,
                   h: int = 4096, n_slots: int = 32, rank: int = 16,
                   draw_w: bool = True) -> Workload:
    """64 decode tokens, ids ~ finite Zipf(1.1) over 32 slots, rank 16, 4096->4096.

    bf16; x ~ N(0,1); W, A, B ~ N(0, 0.02); scale = alpha/r = 32/16.
    ``n_modules`` > 1 gives that many independent module instances of the same
    shape (their own x, W, y0 and adapter weights), for one-launch batches."""
    rng = np.random.default_rng(seed)
    ids = zipf_ids(rng, n_tokens, n_slots, 1.1)
    mods = [Module(f"m{i}", h, h, i) for i in range(n_modules)]
    xs, Ws, ad, y0 = _draw_values(rng, "bf16", n_tokens, mods, n_modules,
                                  [[rank] * n_modules] * n_slots,
                                  [32.0 / rank] * n_slots, 1.0, 0.02, 0.02, draw_w)
    return Workload("c2_bgmv_decode", "bf16", h, n_slots, mods, ids, xs, y0, Ws, ad)


# --------------------------------------------------------------------------
# C3: SGMV prefill, q,k,v,o
# --------------------------------------------------------------------------
def c3_sgmv_prefill(seed: int = 3, h: int = 4096, n_slots: int = 8, rank: int = 16,
                    units: Tuple[int, int] = (8, 64), total_units: int = 256,
                    unit_tokens: int = 16, draw_w: bool = True) -> Workload:
    """8 segments, lengths 16*u with u iid uniform in {8..64} conditioned on sum 256
    (rejection sampling), so lengths lie in [128, 1024], are multiples of 16 and
    total 4096 tokens.  Segment slots are a permutation of 0..7.  Modules q,k,v
    share one x; o has its own.  bf16, values as the decode workload."""
    rng = np.random.default_rng(seed)
    while True:
        u = rng.integers(units[0], units[1] + 1, n_slots)
        if int(u.sum()) == total_units:
            break
    lengths = u * unit_tokens
    order = rng.permutation(n_slots).astype(np.int32)
    ids = np.repeat(order, lengths).astype(np.int32)
    mods = [Module("q", h, h, 0), Module("k", h, h, 0), Module("v", h, h, 0),
            Module("o", h, h, 1)]
    xs, Ws, ad, y0 = _draw_values(rng, "bf16", ids.shape[0], mods, 2,
                                  [[rank] * 4] * n_slots, [32.0 / rank] * n_slots,
                                  1.0, 0.02, 0.02, draw_w)
    return Workload("c3_sgmv_prefill", "bf16", h, n_slots, mods, ids, xs, y0, Ws, ad,
                    notes={"segment_lengths": lengths, "segment_slots": order})


# --------------------------------------------------------------------------
# C4: mixed rank, prefill segments + decode tokens
# --------------------------------------------------------------------------
def c4_mixed_rank(seed: int = 4, h: int = 4096, n_slots: int = 64,
                  prefill: int = 4, prefill_len: int = 256, decode: int = 48,
                  ranks: Sequence[int] = (8, 16, 32, 64),
                  draw_w: bool = True) -> Workload:
    """64 slots with ranks uniform over {8,16,32,64} and scale 32/r; 4 prefill
    segments of 256 tokens (one id each) then 48 decode tokens (one id each);
    ids ~ finite Zipf(1.0) over 64.  Pages of 4096 elements, bf16."""
    rng = np.random.default_rng(seed)
    slot_rank = rng.choice(np.asarray(ranks), n_slots).astype(int)
    seg_ids = zipf_ids(rng, prefill + decode, n_slots, 1.0)
    ids = np.concatenate([np.repeat(seg_ids[:prefill], prefill_len),
                          seg_ids[prefill:]]).astype(np.int32)
    mods = [Module("proj", h, h, 0)]
    xs, Ws, ad, y0 = _draw_values(rng, "bf16", ids.shape[0], mods, 1,
                                  [[int(r)] for r in slot_rank],
                                  [32.0 / r for r in slot_rank], 1.0, 0.02, 0.02, draw_w)
    return Workload("c4_mixed_rank", "bf16", h, n_slots, mods, ids, xs, y0, Ws, ad,
                    notes={"slot_rank": slot_rank})


# --------------------------------------------------------------------------
# C5: many-adapter encoder step
# --------------------------------------------------------------------------
def c5_encoder_step(seed: int = 5, n_seq: int = 128, seq_len: int = 256,
                    n_slots: int = 1024, rank: int = 16, h: int = 768,
                    ffn: int = 3072, draw_w: bool = True) -> Workload:
    """Encoder layer of width 768: qkv 768->2304, o 768->768, up 768->3072,
    down 3072->768; 1,024 rank-16 adapters all resident in a pool of 768-element
    pages; 128 sequences of 256 tokens with one id per sequence ~ finite
    Zipf(1.2) over 1,024.  Each linear reads its own synthetic x ~ N(0,1);
    W, A, B ~ N(0, 0.02); scale 2; bf16."""
    rng = np.random.default_rng(seed)
    seq_ids = zipf_ids(rng, n_seq, n_slots, 1.2)
    ids = np.repeat(seq_ids, seq_len).astype(np.int32)
    mods = [Module("qkv", h, 3 * h, 0), Module("o", h, h, 1),
            Module("up", h, ffn, 2), Module("down", ffn, h, 3)]
    xs, Ws, ad, y0 = _draw_values(rng, "bf16", ids.shape[0], mods, 4,
                                  [[rank] * 4] * n_slots, [2.0] * n_slots,
                                  1.0, 0.02, 0.02, draw_w)
    return Workload("c5_encoder_step", "bf16", h, n_slots, mods, ids, xs, y0, Ws, ad)


# --------------------------------------------------------------------------
# request traces for the adapter tiers
# --------------------------------------------------------------------------
def lcg_uniforms(seed: int, count: int) -> np.ndarray:
    """``count`` draws in [0, 1) of the 32-bit linear congruential generator
    the study page's cache simulation uses (section "Memory: slots, tiers and
    paging"): state <- (1664525 state + 1013904223) mod 2^32, draw = state / 2^32
    (the state after the step)."""
    out = np.empty(count, dtype=np.float64)
    s = seed & 0xFFFFFFFF
    for i in range(count):
        s = (s * 1664525 + 1013904223) & 0xFFFFFFFF
        out[i] = s / 4294967296.0
    return out


def request_trace(seed: int = 11, n_adapters: int = 500, n_requests: int = 50_000,
                  s: float = 1.1) -> np.ndarray:
    """Adapter id of each request, finite Zipf(s) over ``n_adapters`` (id 0
    hottest), drawn by inverse CDF from ``lcg_uniforms(seed)``: the smallest id
    whose cumulative weight reaches the draw.  The defaults are the study
    page's cache-simulation example (500 adapters, 50,000 requests, s = 1.1,
    seed 11)."""
    cdf = finite_zipf_cdf(n_adapters, s)
    u = lcg_uniforms(seed, n_requests)
    return np.minimum(np.searchsorted(cdf, u, side="left"), n_adapters - 1).astype(np.int32)


def tier_batches(seed: int = 21, n_batches: int = 10, batch: int = 32, n_adapters: int = 12,
                 per_batch: int = 4, h_in: int = 256, h_out: int = 384, page: int = 64) -> Workload:
    """Consecutive decode batches served through adapter tiers: ``n_adapters``
    adapters (ranks 8 and 16, slots indexed by adapter id), each batch of
    ``batch`` tokens draws its tokens' ids from ``per_batch`` adapters picked
    at random (about one token in eight has id -1).  Batch b is tokens
    [b batch, (b+1) batch).  bf16; x ~ N(0,1); W, A, B ~ N(0, 0.02); scale 2."""
    rng = np.random.default_rng(seed)
    ids = []
    for _ in range(n_batches):
        pick = rng.choice(n_adapters, size=per_batch, replace=False)
        b = pick[rng.integers(0, per_batch, size=batch)]
        b[rng.random(batch) < 0.125] = -1
        ids.append(b)
    ids = np.concatenate(ids).astype(np.int32)
    mods = [Module("proj", h_in, h_out, 0)]
    ranks = [[8 if a % 3 == 0 else 16] for a in range(n_adapters)]
    xs, Ws, ad, y0 = _draw_values(rng, "bf16", ids.shape[0], mods, 1, ranks, [2.0] * n_adapters,
                                  1.0, 0.02, 0.02, draw_w=False)
    return Workload("tier_batches", "bf16", page, n_adapters, mods, ids, xs, y0, Ws, ad,
                    notes={"batch": batch})


# --------------------------------------------------------------------------
# fused base + adapter tiles
# --------------------------------------------------------------------------
def fused_tiles(seed: int = 14, h_in: int = 320, h_out: int = 384, page: int = 64,
                decode_tokens: int = 88) -> Workload:
    """Small bf16 workload for the fused base-plus-adapter path: tiles of 256
    tokens with a ragged last tile, a ragged last column tile (384 = 256 + 128),
    12 slots of ranks 1..64 in 64-element pages (several 16-row units per
    adapter), and three token regions:
      tokens   0..255: one run of slot 1 (rank 16);
      tokens 256..511: runs of slot 3 (rank 32) x 100, id -1 x 30, slot 5
                       (rank 64) x 60, slot 0 (rank 8) x 66;
      tokens 512..   : per-token ids uniform over {-1, 0..11, 12} (12 is out
                       of range), like decode tokens.
    x ~ N(0,1); W ~ N(0, 0.005) so that the adapter term is a large share of
    y; A, B ~ N(0, 0.02); scale 32/r; bf16."""
    rng = np.random.default_rng(seed)
    ranks = [8, 16, 24, 32, 48, 64, 16, 16, 5, 1, 40, 16]
    n_slots = len(ranks)
    ids = np.concatenate([
        np.full(256, 1), np.full(100, 3), np.full(30, -1), np.full(60, 5), np.full(66, 0),
        rng.integers(-1, n_slots + 1, size=decode_tokens)]).astype(np.int32)
    mods = [Module("proj", h_in, h_out, 0)]
    xs, Ws, ad, y0 = _draw_values(rng, "bf16", ids.shape[0], mods, 1, [[r] for r in ranks],
                                  [32.0 / r for r in ranks], 1.0, 0.005, 0.02)
    return Workload("fused_tiles", "bf16", page, n_slots, mods, ids, xs, y0, Ws, ad)


# --------------------------------------------------------------------------
# FP8 base
# --------------------------------------------------------------------------
E4M3_MAX = 448.0   # largest finite OCP E4M3 magnitude


def to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """float32 values with |a| <= 448 -> OCP E4M3 codes (uint8), rounded to
    nearest, ties to even (torch's float8_e4m3fn conversion on the CPU)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def with_fp8_base(wl: Workload) -> Workload:
    """The workload with an FP8 base: each module's drawn W (its bf16 values)
    quantized per output column, scale_c = max_k |W[k][c]| / 448 (float32; 1
    for an all-zero column), codes = E4M3(W[k][c] / scale_c).  The bf16 W, x,
    ids and adapters are kept; y0 is not used by the fused pass."""
    import copy
    out = copy.copy(wl)
    out.W8, out.W8_scale = [], []
    for m, W in enumerate(wl.W):
        if W is None:
            out.W8.append(None)
            out.W8_scale.append(None)
            continue
        w32 = (np.asarray(W, np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32) \
            if wl.dtype == "bf16" else np.asarray(W, np.float32)
        amax = np.max(np.abs(w32), axis=0)
        scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        q = np.clip(w32 / scale[None, :], -E4M3_MAX, E4M3_MAX)
        out.W8.append(to_e4m3_codes(q))
        out.W8_scale.append(scale)
    out.name = wl.name + "_fp8w"
    return out


def fp8_code_sweep(h: int = 256, page: int = 256, nan_codes: bool = False) -> Workload:
    """Every E4M3 code through the FP8 base: x is the identity (token i is
    e_i, h tokens), W8[k][c] = (k + c) mod 256 and scale 1, so y[i][c] is the
    value of code (i + c) mod 256 exactly.  The two NaN codes (0x7F, 0xFF) are
    replaced by 0x00 unless nan_codes (a NaN in W reaches every token through
    the zero products).  No adapters (ids -1)."""
    k = np.arange(h)[:, None]
    c = np.arange(h)[None, :]
    codes = ((k + c) % 256).astype(np.uint8)
    if not nan_codes:
        codes[(codes == 0x7F) | (codes == 0xFF)] = 0
    x = to_bf16_bits(np.eye(h, dtype=np.float32))
    mods = [Module("proj", h, h, 0)]
    wl = Workload("fp8_code_sweep", "bf16", page, 1, mods, np.full(h, -1, np.int32), [x],
                  [to_bf16_bits(np.zeros((h, h), np.float32))], [None], [[None]])
    wl.W8 = [codes]
    wl.W8_scale = [np.ones(h, np.float32)]
    return wl


# --------------------------------------------------------------------------
# special inputs used by pins
# --------------------------------------------------------------------------
def fingerprint_rank1(seed: int = 11, n_tokens: int = 96, h: int = 256,
                      n_slots: int = 12, dtype: str = "bf16") -> Workload:
    """Rank-1 adapters A_a = e_{j_a}, B_a = e_{k_a}, scale 1, y0 = 0.

    Every token's adapter term is x_i[j_a] placed in column k_a only, so each
    output row names the adapter it gathered.  (j_a, k_a) are distinct per slot.
    ids mix runs and single tokens, with some -1."""
    rng = np.random.default_rng(seed)
    js = rng.choice(h, n_slots, replace=False)
    ks = rng.choice(h, n_slots, replace=False)
    ids = rng.integers(-1, n_slots, n_tokens).astype(np.int32)
    # a few runs so that segments of several tokens appear
    ids[10:30] = 3
    ids[50:53] = 0
    x = _store(_normal(rng, 1.0, (n_tokens, h)), dtype)
    ad = []
    for s in range(n_slots):
        A = np.zeros((1, h), np.float32); A[0, js[s]] = 1.0
        B = np.zeros((1, h), np.float32); B[0, ks[s]] = 1.0
        ad.append([(1, 1.0, _store(A, dtype), _store(B, dtype))])
    y0 = [_store(np.zeros((n_tokens, h), np.float32), dtype)]
    return Workload("fingerprint_rank1", dtype, h, n_slots, [Module("proj", h, h, 0)],
                    ids, [x], y0, [None], ad, notes={"j": js, "k": ks})


def integer_exact(seed: int = 12, n_tokens: int = 80, h: int = 64, n_slots: int = 6,
                  max_rank: int = 4, dtype: str = "f32", scale: float = 2.0,
                  ranks: Optional[Sequence[int]] = None) -> Workload:
    """Small-integer inputs: x, W, A, B, y0 in {-4..4}, h = 64, rank <= 4, scale 2.

    Every partial sum stays an integer below 2^24, so any fp32 summation order
    gives the exact result."""
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, n_slots, n_tokens).astype(np.int32)
    ids[5:25] = 1
    if ranks is None:
        ranks = [int(r) for r in rng.integers(1, max_rank + 1, n_slots)]

    def ints(shape):
        return rng.integers(-4, 5, shape).astype(np.float32)

    x = _store(ints((n_tokens, h)), dtype)
    W = _store(ints((h, h)), dtype)
    ad = []
    for s in range(n_slots):
        ad.append([(int(ranks[s]), float(scale), _store(ints((ranks[s], h)), dtype),
                    _store(ints((ranks[s], h)), dtype))])
    y0 = [_store(ints((n_tokens, h)), dtype)]
    return Workload("integer_exact", dtype, h, n_slots, [Module("proj", h, h, 0)],
                    ids, [x], y0, [W], ad)


BY_NAME = {
    "c1": c1_tiny_f32,
    "c2": c2_bgmv_decode,
    "c3": c3_sgmv_prefill,
    "c4": c4_mixed_rank,
    "c5": c5_encoder_step,
}
