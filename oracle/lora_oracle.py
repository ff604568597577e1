"""CPU oracle for the multi-LoRA apply path.  TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check of ``__graft_entry__`` and the CPU
baseline leg of ``bench.py`` may import this module.  The GPU library never
calls it and shares no code with it; the only code both sides use is the
seeded input generator in ``workloads`` (random draws, no arithmetic of the
method).

What it computes (fp64, from the exact upcast of the stored input bits):

* The adapted linear layer of the "Multi-LoRA Serving - S-LoRA/Punica
  Batching" study page, section "The kernel trick: gather, do not merge":
  request i with adapter a(i) gets  y_i = x_i W + scale_a (x_i A_a^T) B_a,
  with A_a stored as rank rows of length h_in and B_a stored as rank rows of
  length h_out (the page's B_a transposed).  The slide deck "Thousands of
  adapters" (slide 5) states the same update as xAB added to the shared xW.
* Tokens with adapter id -1 carry no adapter (y_i = x_i W).  Ids outside
  [-1, n_slots) are treated as -1 and counted as bad.  A slot with no adapter
  loaded for a module contributes nothing.
* The segment structure of a batch: tokens grouped by adapter in ascending
  slot order, original order kept inside a group (a stable sort), tokens
  without an adapter dropped.  This is the grouping step of the Fastino
  article ("groups a batch's tokens by adapter") and of SGMV's "contiguous
  segments of tokens sharing an adapter" on the study page.

Every function loops over tokens one by one; the only library routines used
are fp64 dot/matrix-vector products and a stable argsort.
"""
from __future__ import annotations

from typing import Dict, Iterable, Optional, Sequence

import numpy as np

__all__ = [
    "decode", "decode_e4m3", "adapter_term", "lora_delta", "base_product", "lora_forward",
    "apply_to_y0", "merged_forward", "build_segments", "shrink_t",
    "base_product_fp8w", "lora_forward_fp8w",
]


# --------------------------------------------------------------------------
# exact upcast of stored values
# --------------------------------------------------------------------------
def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64, exactly.  bf16 bits widen to float32 by a
    16-bit left shift (the bfloat16 format is the top half of binary32)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) -> float64, exactly, from the format's
    definition: bit 7 is the sign, bits 6..3 the exponent e (bias 7), bits 2..0
    the mantissa m.  e >= 1: (1 + m/8) 2^(e-7) = (8 + m) 2^(e-10); e = 0: the
    subnormals m 2^-9 (and +-0); e = 15 with m = 7 is NaN; there are no
    infinities, so the largest finite magnitude is 448 (e = 15, m = 6)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    mag = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp((8 + m).astype(np.float64), (e - 10).astype(np.int64)))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


def _adapter(wl, slot: int, module: int):
    """(rank, scale, A, B) in float64 for an in-range slot, else None."""
    if slot < 0 or slot >= wl.n_slots:
        return None
    a = wl.adapters[slot][module]
    if a is None:
        return None
    rank, scale, A, B = a
    return rank, float(scale), decode(A, wl.dtype), decode(B, wl.dtype)


# --------------------------------------------------------------------------
# the adapter term of one token
# --------------------------------------------------------------------------
def adapter_term(x_row: np.ndarray, A: np.ndarray, B: np.ndarray, scale: float):
    """scale * (x A^T) B for one token, plus the intermediate t = x A^T.

    Study page, "The kernel trick": the "shrink" x_i A_a^T gives r numbers per
    token, the "expand" multiplies them into B_a, and the result is scaled."""
    t = A @ x_row                 # [r]: one dot product per rank row
    return scale * (t @ B), t     # [h_out]


def _tokens(wl, tokens: Optional[Iterable[int]]):
    return range(wl.n_tokens) if tokens is None else list(tokens)


def lora_delta(wl, module: int, tokens: Optional[Iterable[int]] = None) -> np.ndarray:
    """Adapter term for each requested token of ``module``: [len(tokens), h_out]."""
    mod = wl.modules[module]
    x = wl.x[mod.x_group]
    toks = _tokens(wl, tokens)
    out = np.zeros((len(toks), mod.h_out), dtype=np.float64)
    cache: Dict[int, object] = {}
    for row, i in enumerate(toks):
        a = int(wl.ids[i])
        if a not in cache:
            cache[a] = _adapter(wl, a, module)
        ad = cache[a]
        if ad is None:
            continue
        rank, scale, A, B = ad
        out[row], _ = adapter_term(decode(x[i], wl.dtype), A, B, scale)
    return out


def shrink_t(wl, module: int, tokens: Optional[Iterable[int]] = None):
    """t = x_i A_a^T per requested token (NaN where the token has no adapter).

    Returns an array [len(tokens), max_rank]; entries past the adapter's rank
    are NaN as well."""
    mod = wl.modules[module]
    x = wl.x[mod.x_group]
    toks = _tokens(wl, tokens)
    out = np.full((len(toks), wl.max_rank()), np.nan)
    for row, i in enumerate(toks):
        ad = _adapter(wl, int(wl.ids[i]), module)
        if ad is None:
            continue
        rank, scale, A, B = ad
        _, t = adapter_term(decode(x[i], wl.dtype), A, B, scale)
        out[row, :rank] = t
    return out


def base_product(wl, module: int, tokens: Optional[Iterable[int]] = None) -> np.ndarray:
    """The shared base product x_i W for each requested token (fp64)."""
    mod = wl.modules[module]
    x = wl.x[mod.x_group]
    W = decode(wl.W[module], wl.dtype)
    toks = _tokens(wl, tokens)
    out = np.empty((len(toks), mod.h_out), dtype=np.float64)
    for row, i in enumerate(toks):
        out[row] = decode(x[i], wl.dtype) @ W
    return out


def lora_forward(wl, module: int, tokens: Optional[Iterable[int]] = None) -> np.ndarray:
    """y_i = x_i W + scale_a (x_i A_a^T) B_a for each requested token."""
    return base_product(wl, module, tokens) + lora_delta(wl, module, tokens)


def base_product_fp8w(wl, module: int, tokens: Optional[Iterable[int]] = None) -> np.ndarray:
    """The base product with an FP8 base (the study page's "Operating it":
    a quantized base under bf16 adapters): x_i W with W[k][c] =
    w_scale[c] * E(W8[k][c]), E the exact value of an E4M3 code and w_scale
    one float32 scale per output column.  fp64 per token."""
    mod = wl.modules[module]
    x = wl.x[mod.x_group]
    W = decode_e4m3(wl.W8[module]) * np.asarray(wl.W8_scale[module], np.float32).astype(np.float64)[None, :]
    toks = _tokens(wl, tokens)
    out = np.empty((len(toks), mod.h_out), dtype=np.float64)
    for row, i in enumerate(toks):
        out[row] = decode(x[i], wl.dtype) @ W
    return out


def lora_forward_fp8w(wl, module: int, tokens: Optional[Iterable[int]] = None) -> np.ndarray:
    """y_i = x_i W (FP8 base, base_product_fp8w) + scale_a (x_i A_a^T) B_a."""
    return base_product_fp8w(wl, module, tokens) + lora_delta(wl, module, tokens)


def apply_to_y0(wl, module: int, tokens: Optional[Iterable[int]] = None) -> np.ndarray:
    """y0_i + adapter term: what the library leaves in a buffer that held y0."""
    toks = _tokens(wl, tokens)
    y0 = decode(wl.y0[module][np.asarray(list(toks), dtype=np.int64)], wl.dtype)
    return y0 + lora_delta(wl, module, toks)


def merged_forward(wl, module: int, tokens: Optional[Iterable[int]] = None) -> np.ndarray:
    """The merged-weight form: for each distinct adapter build W' = W + s A^T B
    and multiply its tokens by it (option 1 of the study page's demo; slide 5 of
    "Thousands of adapters": W' = W + AB).  Tokens without an adapter use W."""
    mod = wl.modules[module]
    x = wl.x[mod.x_group]
    W = decode(wl.W[module], wl.dtype)
    toks = _tokens(wl, tokens)
    out = np.empty((len(toks), mod.h_out), dtype=np.float64)
    merged: Dict[int, np.ndarray] = {}
    for row, i in enumerate(toks):
        a = int(wl.ids[i])
        if a not in merged:
            ad = _adapter(wl, a, module)
            if ad is None:
                merged[a] = W
            else:
                rank, scale, A, B = ad
                merged[a] = W + scale * (A.T @ B)
        out[row] = decode(x[i], wl.dtype) @ merged[a]
    return out


# --------------------------------------------------------------------------
# segments
# --------------------------------------------------------------------------
def build_segments(ids: Sequence[int], n_slots: int) -> Dict[str, object]:
    """Group token indices by adapter slot.

    perm      token indices with a valid id, sorted by id, original order kept
              within an id (stable sort)
    seg_start offsets of each group in perm, plus the total at the end
    seg_slot  the slot of each group, ascending
    n_bad     ids outside [-1, n_slots)
    """
    ids = np.asarray(ids, dtype=np.int64)
    valid = (ids >= 0) & (ids < n_slots)
    n_bad = int(np.count_nonzero((ids < -1) | (ids >= n_slots)))
    order = np.argsort(ids, kind="stable")
    perm = order[valid[order]].astype(np.int32)
    slots, counts = np.unique(ids[perm], return_counts=True)
    seg_start = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return {
        "perm": perm,
        "seg_start": seg_start,
        "seg_slot": slots.astype(np.int32),
        "n_seg": int(slots.shape[0]),
        "n_active": int(perm.shape[0]),
        "max_seg_len": int(counts.max()) if counts.size else 0,
        "n_bad": n_bad,
    }
