"""Asynchronous lora_pool_load (GPU; C ABI): the call returns before the upload
completes ("Thousands of adapters", slide 9: copies overlap the GPU's work),
with host sources copied into a page-locked staging ring before it returns.

* load -> apply -> evict -> load another adapter into the freed pages -> apply,
  all enqueued on one stream with no synchronization in between: both applies
  equal the oracle bit for bit (integer inputs, fp32);
* a host buffer overwritten right after each of 11 loads (more than the ring's
  4 slots): every entry reads back the values it had at its call;
* device-memory sources, read on the stream.
"""
import numpy as np
import pytest

import workloads as W
from oracle import lora_oracle as lo
from gpu_util import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import segmented_gathered_rank_amd as sgr  # noqa: E402
from segmented_gathered_rank_amd.harness import DeviceWorkload, from_device  # noqa: E402


def _read(pool, slot, module, rank, h_in, h_out):
    A = np.zeros((rank, h_in), np.float32)
    B = np.zeros((rank, h_out), np.float32)
    r, sc, _ = sgr.lora_pool_read(pool, slot, module, A, B)
    return r, sc, A, B


def test_load_apply_evict_reload_on_one_stream():
    wl = W.integer_exact(seed=51, n_tokens=96, n_slots=6, ranks=[2, 3, 4, 1, 4, 3])
    rng = np.random.default_rng(52)
    dw = DeviceWorkload(wl, load=True, extra_pages=64)
    torch.cuda.synchronize()
    # slot 4 gets a fresh adapter X, then is evicted and reloaded with Y into the same pages
    h = wl.modules[0].h_in
    X = (4, 2.0, rng.integers(-4, 5, (4, h)).astype(np.float32), rng.integers(-4, 5, (4, h)).astype(np.float32))
    Y = (3, 2.0, rng.integers(-4, 5, (3, h)).astype(np.float32), rng.integers(-4, 5, (3, h)).astype(np.float32))
    ys = []
    sgr.lora_pool_evict(dw.pool, 4)
    for ad in (X, Y):
        r, sc, A, B = ad
        sgr.lora_pool_load(dw.pool, 4, 0, r, A, B, sc)    # returns before the upload is done
        dw.reset_y()
        dw.build_segments()
        dw.bgmv()
        ys.append(dw.y_of(0).clone())
        sgr.lora_pool_evict(dw.pool, 4)
    torch.cuda.synchronize()
    for ad, y in zip((X, Y), ys):
        wl.adapters[4] = [ad]
        assert np.array_equal(y.cpu().numpy(), lo.apply_to_y0(wl, 0)), f"rank {ad[0]}"
    dw.close()


def test_host_buffer_reused_right_after_each_load():
    wl = W.integer_exact(seed=53, n_tokens=8, n_slots=12, ranks=[4] * 12)
    dw = DeviceWorkload(wl, load=False)
    mods = wl.modules
    dw.pool = sgr.lora_pool_create(0, sgr.LORA_F32, wl.page_elems, 200, 12, 1, [mods[0].h_in], [mods[0].h_out], 4)
    h = mods[0].h_in
    bufA = np.zeros((4, h), np.float32)
    bufB = np.zeros((4, h), np.float32)
    expect = {}
    for s in range(11):
        bufA[:] = s + 1
        bufB[:] = -(s + 1)
        sgr.lora_pool_load(dw.pool, s, 0, 4, bufA, bufB, 1.0)
        expect[s] = (bufA.copy(), bufB.copy())
        bufA[:] = 999.0                                   # overwritten before the upload ran
        bufB[:] = 999.0
    for s in range(11):
        r, sc, A, B = _read(dw.pool, s, 0, 4, h, h)
        assert r == 4 and np.array_equal(A, expect[s][0]) and np.array_equal(B, expect[s][1]), s
    dw.close()


def test_device_sources():
    wl = W.integer_exact(seed=54, n_tokens=8, n_slots=4, ranks=[3] * 4)
    dw = DeviceWorkload(wl, load=False)
    h = wl.modules[0].h_in
    dw.pool = sgr.lora_pool_create(0, sgr.LORA_F32, wl.page_elems, 64, 4, 1, [h], [h], 3)
    rng = np.random.default_rng(55)
    vals = []
    for s in range(4):
        A = rng.integers(-4, 5, (3, h)).astype(np.float32)
        B = rng.integers(-4, 5, (3, h)).astype(np.float32)
        dA, dB = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        sgr.lora_pool_load(dw.pool, s, 0, 3, dA, dB if s % 2 else B, 0.5)   # device A; device or host B
        vals.append((A, B, dA, dB))
    torch.cuda.synchronize()
    for s, (A, B, _, _) in enumerate(vals):
        r, sc, rA, rB = _read(dw.pool, s, 0, 3, h, h)
        assert r == 3 and sc == 0.5 and np.array_equal(rA, A) and np.array_equal(rB, B), s
    say("device sources read back")
    dw.close()
