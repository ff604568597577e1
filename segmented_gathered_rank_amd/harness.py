"""Host-side driver: uploads a workload and issues the library's calls.

Used by the tests, the benchmark and the smoke check.  It only moves data
(numpy -> device tensors, adapters -> pool pages) and sequences C-ABI calls;
every step of the apply path runs in the HIP library.

A workload is any object with the attributes of ``workloads.Workload``:
dtype, page_elems, n_slots, modules (h_in, h_out, x_group), ids, x, y0 and
adapters[slot][module] = (rank, scale, A, B) or None.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np
import torch

from . import (LORA_BF16, LORA_F32, lora_apply_bgmv, lora_apply_bgmv_ids, lora_apply_bgmv_packed, lora_apply_sgmv, lora_apply_sgmv_multi,
               lora_build_segments, lora_expand,
               lora_fused_gemm, lora_fused_gemm_fp8w,
               lora_pool_create, lora_pool_destroy, lora_pool_load, lora_segments_bind,
               lora_segments_bytes, lora_shrink, lora_shrink_workspace_bytes)

__all__ = ["DeviceWorkload", "to_device", "from_device"]


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Storage array (float32, or uint16 bf16 bits) -> device tensor, bits unchanged."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def from_device(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> storage array (float32, or uint16 bf16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DeviceWorkload:
    """A workload resident on one GPU: pool, x, y (= y0 copies), t, segments."""

    def __init__(self, wl, device: int = 0, n_pages: Optional[int] = None, y_dtype: Optional[str] = None,
                 extra_pages: int = 0, max_rank: Optional[int] = None, load: bool = True):
        self.wl = wl
        self.dev = torch.device("cuda", device)
        self.dtype = wl.dtype
        self.y_dtype = y_dtype or wl.dtype
        n = wl.n_tokens
        self.n = n
        mods = wl.modules
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        ydt = torch.bfloat16 if self.y_dtype == "bf16" else torch.float32
        self.max_rank = max_rank or wl.max_rank()
        self.ld_t = max(16, (self.max_rank + 3) // 4 * 4)

        # x: one flat tensor, every x group at a known element offset
        self.x_off = []
        sizes = [int(np.prod(a.shape)) for a in wl.x]
        self.x = torch.empty(max(1, sum(sizes)), dtype=tdt, device=self.dev)
        off = 0
        for g, a in enumerate(wl.x):
            self.x[off:off + sizes[g]] = to_device(a, wl.dtype, self.dev).reshape(-1)
            self.x_off.append(off)
            off += sizes[g]

        # shape groups: consecutive modules with equal (h_in, h_out) share one y and one t tensor
        self.groups: List[Tuple[int, int]] = []
        m = 0
        while m < len(mods):
            e = m + 1
            while e < len(mods) and (mods[e].h_in, mods[e].h_out) == (mods[m].h_in, mods[m].h_out):
                e += 1
            self.groups.append((m, e))
            m = e
        self.y = []
        for (m0, m1) in self.groups:
            self.y.append(torch.empty((m1 - m0, n, mods[m0].h_out), dtype=ydt, device=self.dev))
        # shrink groups: consecutive modules with equal h_in, one shrink call each (t of all
        # modules is one tensor, so any run of modules has a uniform t stride)
        self.in_groups: List[Tuple[int, int]] = []
        m = 0
        while m < len(mods):
            e = m + 1
            while e < len(mods) and mods[e].h_in == mods[m].h_in:
                e += 1
            self.in_groups.append((m, e))
            m = e
        self.t = torch.zeros((len(mods), n, self.ld_t), dtype=torch.float32, device=self.dev)
        self.reset_y()

        self.pool = None
        if load:
            self.pool = lora_pool_create(device, LORA_BF16 if wl.dtype == "bf16" else LORA_F32,
                                         wl.page_elems, (n_pages or wl.pages_needed()) + extra_pages,
                                         wl.n_slots, len(mods), [m.h_in for m in mods],
                                         [m.h_out for m in mods], self.max_rank)
            self.load_all()
        self.ids = torch.from_numpy(np.ascontiguousarray(wl.ids, dtype=np.int32)).to(self.dev)
        nb = lora_segments_bytes(n, wl.n_slots)
        self.seg_buf = torch.zeros(max(nb, 256), dtype=torch.uint8, device=self.dev)
        self.seg = lora_segments_bind(self.seg_buf, n, wl.n_slots)
        self.ws_bytes = max(lora_shrink_workspace_bytes(self.pool, n, len(mods)) if self.pool else 0, 16)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=self.dev)

    # ---------------------------------------------------------------- data
    def load_all(self):
        for s, row in enumerate(self.wl.adapters):
            for m, a in enumerate(row):
                if a is not None:
                    rank, scale, A, B = a
                    lora_pool_load(self.pool, s, m, rank, np.ascontiguousarray(A), np.ascontiguousarray(B),
                                   scale)
        torch.cuda.synchronize(self.dev)

    def reset_y(self):
        """y <- y0 (converted to the output dtype if it differs)."""
        for gi, (m0, m1) in enumerate(self.groups):
            for m in range(m0, m1):
                y0 = to_device(self.wl.y0[m], self.wl.dtype, self.dev)
                self.y[gi][m - m0].copy_(y0.to(self.y[gi].dtype))

    def zero_y(self):
        for y in self.y:
            y.zero_()

    def y_of(self, module: int) -> torch.Tensor:
        for gi, (m0, m1) in enumerate(self.groups):
            if m0 <= module < m1:
                return self.y[gi][module - m0]
        raise IndexError(module)

    def t_of(self, module: int) -> torch.Tensor:
        return self.t[module]

    # ---------------------------------------------------------------- calls
    def _x_runs(self, m0: int, m1: int):
        """Split modules [m0, m1) into runs whose x offsets step uniformly."""
        mods = self.wl.modules
        runs, m = [], m0
        while m < m1:
            e = m + 1
            xo = self.x_off[mods[m].x_group]
            stride = None
            while e < m1:
                d = self.x_off[mods[e].x_group] - self.x_off[mods[e - 1].x_group]
                if stride is None:
                    stride = d
                if d != stride or d < 0:
                    break
                e += 1
            runs.append((m, e, xo, stride or 0))
            m = e
        return runs

    def _xp(self, off: int) -> int:
        return self.x.data_ptr() + off * self.x.element_size()

    def build_segments(self, stream=None):
        lora_build_segments(self.ids, self.seg, stream)

    def shrink(self, stream=None):
        mods = self.wl.modules
        t = self.t
        for (m0, m1) in self.in_groups:
            h_in = mods[m0].h_in
            for (a, b, xo, msx) in self._x_runs(m0, m1):
                lora_shrink(self.pool, a, b - a, self._xp(xo), h_in, msx, self.seg, t[a], self.ld_t, t.stride(0),
                            self.ws, self.ws_bytes, stream)

    def expand(self, stream=None):
        ydt = LORA_BF16 if self.y_dtype == "bf16" else LORA_F32
        mods = self.wl.modules
        t = self.t
        for gi, (m0, m1) in enumerate(self.groups):
            y = self.y[gi]
            lora_expand(self.pool, m0, m1 - m0, t[m0], self.ld_t, t.stride(0), self.seg, y, mods[m0].h_out,
                        y.stride(0), ydt, stream)

    def sgmv(self, stream=None):
        """Shrink and expand through lora_apply_sgmv (one x run) or lora_apply_sgmv_multi
        (several: q, k, v sharing x beside o): one call per run of modules of one shape."""
        ydt = LORA_BF16 if self.y_dtype == "bf16" else LORA_F32
        mods = self.wl.modules
        t = self.t
        for gi, (m0, m1) in enumerate(self.groups):
            y = self.y[gi]
            h_in, h_out = mods[m0].h_in, mods[m0].h_out
            runs = self._x_runs(m0, m1)
            if len(runs) == 1:
                a, b, xo, msx = runs[0]
                lora_apply_sgmv(self.pool, a, b - a, self._xp(xo), h_in, msx, self.seg, t[a], self.ld_t,
                                t.stride(0), y, h_out, y.stride(0), ydt, self.ws, self.ws_bytes, stream)
            else:
                lora_apply_sgmv_multi(self.pool, m0, m1 - m0, [(self._xp(xo), h_in, msx, b - a)
                                                               for (a, b, xo, msx) in runs],
                                      self.seg, t[m0], self.ld_t, t.stride(0), y, h_out, y.stride(0), ydt,
                                      self.ws, self.ws_bytes, stream)

    def sgmv_fused_calls(self) -> bool:
        """Whether apply() takes the combined calls: when the modules have one shape (one
        call covers the step).  Modules of several shapes (an encoder layer's qkv, o,
        up and down) are better served by lora_shrink over each run of equal h_in and
        lora_expand over each shape."""
        return len(self.groups) == 1

    def apply(self, stream=None):
        """The adapter term of every module added to y: lora_apply_sgmv calls where
        sgmv_fused_calls() holds, else lora_shrink and lora_expand calls."""
        if self.sgmv_fused_calls():
            self.sgmv(stream)
        else:
            self.shrink(stream)
            self.expand(stream)

    def bgmv(self, stream=None):
        ydt = LORA_BF16 if self.y_dtype == "bf16" else LORA_F32
        mods = self.wl.modules
        for gi, (m0, m1) in enumerate(self.groups):
            y = self.y[gi]
            for (a, b, xo, msx) in self._x_runs(m0, m1):
                yp = y.data_ptr() + (a - m0) * y.stride(0) * y.element_size()
                lora_apply_bgmv(self.pool, a, b - a, self._xp(xo), mods[m0].h_in, msx, self.seg, yp,
                                mods[m0].h_out, y.stride(0), ydt, stream)

    def bgmv_ids(self, stream=None):
        """As bgmv(), straight from the ids (lora_apply_bgmv_ids: no segment build; <= 64 tokens)."""
        ydt = LORA_BF16 if self.y_dtype == "bf16" else LORA_F32
        mods = self.wl.modules
        for gi, (m0, m1) in enumerate(self.groups):
            y = self.y[gi]
            for (a, b, xo, msx) in self._x_runs(m0, m1):
                yp = y.data_ptr() + (a - m0) * y.stride(0) * y.element_size()
                lora_apply_bgmv_ids(self.pool, a, b - a, self._xp(xo), mods[m0].h_in, msx, self.ids, self.n, yp,
                                    mods[m0].h_out, y.stride(0), ydt, stream)

    def bgmv_packed(self, stream=None):
        """As bgmv(), with runs of 2..4 modules that share x through lora_apply_bgmv_packed."""
        ydt = LORA_BF16 if self.y_dtype == "bf16" else LORA_F32
        mods = self.wl.modules
        for gi, (m0, m1) in enumerate(self.groups):
            y = self.y[gi]
            for (a, b, xo, msx) in self._x_runs(m0, m1):
                yp = y.data_ptr() + (a - m0) * y.stride(0) * y.element_size()
                if msx == 0 and 2 <= b - a <= 4:
                    lora_apply_bgmv_packed(self.pool, a, b - a, self._xp(xo), mods[m0].h_in, self.seg, yp,
                                           mods[m0].h_out, y.stride(0), ydt, stream)
                else:
                    lora_apply_bgmv(self.pool, a, b - a, self._xp(xo), mods[m0].h_in, msx, self.seg, yp,
                                    mods[m0].h_out, y.stride(0), ydt, stream)

    def upload_weights(self):
        """W^T of every module ([h_out][h_in], the layout lora_fused_gemm reads)."""
        self.wT = []
        for m in range(len(self.wl.modules)):
            W = self.wl.W[m]
            self.wT.append(None if W is None else to_device(np.ascontiguousarray(W.T), self.wl.dtype, self.dev))

    def fused(self, stream=None, adapters: bool = True, modules=None):
        """y = x W (+ the adapter term) per module in one lora_fused_gemm call each."""
        mods = self.wl.modules
        if not hasattr(self, "wT"):
            self.upload_weights()
        for m in (range(len(mods)) if modules is None else modules):
            h_in, h_out = mods[m].h_in, mods[m].h_out
            lora_fused_gemm(self.pool, m, self._xp(self.x_off[mods[m].x_group]), h_in, self.wT[m], h_in,
                            self.ids if adapters else None, self.n, self.y_of(m), h_out, stream)

    def upload_weights_fp8(self):
        """W^T as E4M3 codes ([h_out][h_in] bytes) and the column scales of every module."""
        self.w8T, self.w8s = [], []
        for m in range(len(self.wl.modules)):
            W8 = self.wl.W8[m]
            if W8 is None:
                self.w8T.append(None)
                self.w8s.append(None)
                continue
            self.w8T.append(torch.from_numpy(np.ascontiguousarray(W8.T)).to(self.dev))
            self.w8s.append(torch.from_numpy(np.ascontiguousarray(self.wl.W8_scale[m], np.float32)).to(self.dev))

    def fused_fp8(self, stream=None, adapters: bool = True, modules=None):
        """y = x W (FP8 base) (+ the adapter term) per module in one lora_fused_gemm_fp8w call each."""
        mods = self.wl.modules
        if not hasattr(self, "w8T"):
            self.upload_weights_fp8()
        for m in (range(len(mods)) if modules is None else modules):
            h_in, h_out = mods[m].h_in, mods[m].h_out
            lora_fused_gemm_fp8w(self.pool, m, self._xp(self.x_off[mods[m].x_group]), h_in, self.w8T[m], h_in,
                                 self.w8s[m], self.ids if adapters else None, self.n, self.y_of(m), h_out, stream)

    def sgmv_step(self, stream=None):
        self.build_segments(stream)
        self.apply(stream)

    def bgmv_step(self, stream=None):
        self.build_segments(stream)
        self.bgmv(stream)

    def close(self):
        if self.pool is not None:
            torch.cuda.synchronize(self.dev)
            lora_pool_destroy(self.pool)
            self.pool = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
