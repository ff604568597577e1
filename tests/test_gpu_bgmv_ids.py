"""Fused BGMV straight from the ids (GPU; C ABI): lora_apply_bgmv_ids builds a
decode batch's unit list inside every workgroup instead of in a segment-build
launch (study page, "The kernel trick": each decode token brings its own
adapter index).

* the same y bits as lora_build_segments + lora_apply_bgmv, one module and the
  grouped launch over 128 modules, bf16 and fp32 outputs, an fp32 pool;
* exact sums: integer inputs and rank-1 fingerprints against the oracle;
* edges: 0 tokens (nothing written), 1 token, 64 tokens of one id (a segment
  long enough for a matrix-core tile), ids -1 and out of range (rows left as
  they were), 65 tokens (SHAPE, nothing launched);
* the decode batch of 64 tokens over q, k, v, o of 4096 x 4096 against the oracle;
* one module of 4096 columns, whose units run as column ranges: exact sums, both paths.
"""
import dataclasses

import numpy as np
import pytest

import workloads as W
from oracle import lora_oracle as lo
from gpu_util import assert_close, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import segmented_gathered_rank_amd as sgr  # noqa: E402
from segmented_gathered_rank_amd.harness import DeviceWorkload, from_device  # noqa: E402


def _bits(t):
    a = from_device(t)
    return a.view(np.uint16 if a.dtype == np.float16 or a.itemsize == 2 else np.uint32).copy()


def _both_paths(wl, **kw):
    """y after build + lora_apply_bgmv, and after lora_apply_bgmv_ids, from the same y0."""
    dw = DeviceWorkload(wl, **kw)
    dw.bgmv_step()
    torch.cuda.synchronize()
    ref = [_bits(dw.y_of(m)) for m in range(wl.n_modules)]
    dw.reset_y()
    dw.bgmv_ids()
    torch.cuda.synchronize()
    got = [_bits(dw.y_of(m)) for m in range(wl.n_modules)]
    return dw, ref, got


@pytest.mark.parametrize("n_modules,y_dtype", [(1, None), (1, "f32"), (128, None)])
def test_same_bits_as_segments_path(n_modules, y_dtype):
    wl = W.c2_bgmv_decode(n_modules=n_modules, h=1024 if n_modules > 1 else 4096, draw_w=False)
    say(f"ids vs segments: {n_modules} modules, y {y_dtype or 'bf16'}")
    dw, ref, got = _both_paths(wl, y_dtype=y_dtype)
    for m in range(wl.n_modules):
        assert np.array_equal(ref[m], got[m]), m
    dw.close()


def test_fp32_pool_same_bits_and_oracle():
    wl = W.c1_tiny_f32()
    dw, ref, got = _both_paths(wl)
    for m in range(wl.n_modules):
        assert np.array_equal(ref[m], got[m]), m
        assert_close(lo.decode(from_device(dw.y_of(m)), dw.y_dtype), lo.apply_to_y0(wl, m), "f32", f"module {m}")
    dw.close()


@pytest.mark.parametrize("kind", ["integer", "fingerprint"])
def test_exact_sums(kind):
    """Integer inputs and rank-1 one-hot adapters: every sum is exact, so y equals the oracle."""
    if kind == "integer":
        wl = W.integer_exact(n_tokens=64)
    else:
        wl = W.fingerprint_rank1(n_tokens=64, dtype="f32")
    dw = DeviceWorkload(wl)
    dw.bgmv_ids()
    torch.cuda.synchronize()
    for m in range(wl.n_modules):
        got = lo.decode(from_device(dw.y_of(m)), dw.y_dtype)
        assert np.array_equal(got, lo.apply_to_y0(wl, m)), m
    dw.close()


@pytest.mark.parametrize("case", ["one_token", "one_long_segment", "bad_ids"])
def test_edges(case):
    wl = W.c2_bgmv_decode(h=512, draw_w=False)
    if case == "one_token":
        wl = dataclasses.replace(wl, ids=wl.ids[:1].copy(), x=[x[:1].copy() for x in wl.x],
                                 y0=[y[:1].copy() for y in wl.y0])
    elif case == "one_long_segment":
        wl.ids = np.full(64, 7, dtype=np.int32)
    else:
        ids = wl.ids.copy()
        ids[::5] = -1
        ids[3] = wl.n_slots + 4      # outside the pool's slots: row left untouched
        ids[11] = -7
        wl.ids = ids
    say(f"ids edge: {case}")
    dw, ref, got = _both_paths(wl)
    for m in range(wl.n_modules):
        assert np.array_equal(ref[m], got[m]), m
    y = lo.decode(from_device(dw.y_of(0)), dw.y_dtype)
    bad = (wl.ids < 0) | (wl.ids >= wl.n_slots)
    y0 = lo.decode(np.asarray(wl.y0[0]), wl.dtype)
    assert np.array_equal(y[bad], y0[bad])
    dw.close()


def test_empty_and_oversized_batches():
    wl = W.c2_bgmv_decode(h=256, draw_w=False)
    dw = DeviceWorkload(wl)
    before = _bits(dw.y_of(0))
    y = dw.y[0]
    sgr.lora_apply_bgmv_ids(dw.pool, 0, 1, dw._xp(dw.x_off[0]), 256, 0, dw.ids, 0, y[0], 256, 0, sgr.LORA_BF16)
    torch.cuda.synchronize()
    assert np.array_equal(before, _bits(dw.y_of(0)))           # 0 tokens: nothing written
    with pytest.raises(sgr.LoraError) as ei:
        sgr.lora_apply_bgmv_ids(dw.pool, 0, 1, dw._xp(dw.x_off[0]), 256, 0, dw.ids, 65, y[0], 256, 0, sgr.LORA_BF16)
    assert ei.value.status == -2                                  # SHAPE: more than 64 tokens
    with pytest.raises(sgr.LoraError) as ei:
        sgr.lora_apply_bgmv_ids(dw.pool, 0, 1, dw._xp(dw.x_off[0]), 256, 0, None, 4, y[0], 256, 0, sgr.LORA_BF16)
    assert ei.value.status == -1                                  # ARG: no ids
    torch.cuda.synchronize()
    assert np.array_equal(before, _bits(dw.y_of(0)))
    dw.close()


def test_qkvo_decode_full_size():
    """64 decode tokens over 8 adapters of rank 16 on q, k, v, o of 4096 x 4096: every token, bf16 bar."""
    wl = W.c3_sgmv_prefill(draw_w=False)
    rng = np.random.default_rng(78)
    n = 64
    wl.ids = W.zipf_ids(rng, n, wl.n_slots, 1.1)
    wl.x = [x[:n].copy() for x in wl.x]
    wl.y0 = [y[:n].copy() for y in wl.y0]
    say("ids path: q,k,v,o decode 64 tokens, 4096^2")
    dw = DeviceWorkload(wl)
    dw.bgmv_ids()
    torch.cuda.synchronize()
    for m in range(wl.n_modules):
        got = lo.decode(from_device(dw.y_of(m)), "bf16")
        assert_close(got, lo.apply_to_y0(wl, m), "bf16", f"module {m}")
    dw.close()


@pytest.mark.parametrize("path", ["bgmv", "bgmv_ids"])
def test_split_units_exact(path):
    """One module of 4096 columns: the launch splits each unit into 4 column ranges, each
    running the whole shrink; integer inputs make every sum exact, so y equals the oracle."""
    wl = W.integer_exact(n_tokens=64, h=4096)
    dw = DeviceWorkload(wl)
    if path == "bgmv":
        dw.bgmv_step()
    else:
        dw.bgmv_ids()
    torch.cuda.synchronize()
    got = lo.decode(from_device(dw.y_of(0)), dw.y_dtype)
    assert np.array_equal(got, lo.apply_to_y0(wl, 0))
    dw.close()
