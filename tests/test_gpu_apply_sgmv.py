"""lora_apply_sgmv (GPU; C ABI): lora_shrink then lora_expand with the K-split
partial tiles added inside the expand ("Thousands of adapters", slide 11: one
SGMV call for a mixed batch).

The expand adds the splits in the order lora_shrink's own sum does, so y must
equal the two-call path bit for bit on every workload; the oracle comparisons
of the same workloads run through the harness's step (which takes
lora_apply_sgmv for them) in test_gpu_parity.py.  Covered: the prefill and
mixed-rank batches at full size (K split 4 and 8 ways, rank caps 16 and 64), fp32
output, shared-x modules with rank caps 32/48/64 (every partial-tile width),
many modules per launch, fp32 pools (no matrix cores), no workspace (no split),
and argument errors.
"""
import numpy as np
import pytest

import workloads as W
from oracle import lora_oracle as lo
from gpu_util import assert_close, run, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import segmented_gathered_rank_amd as sgr  # noqa: E402
from segmented_gathered_rank_amd.harness import DeviceWorkload, from_device  # noqa: E402


def _both(wl, y_dtype=None, folded=None, **kw):
    """y after lora_apply_sgmv calls and after lora_shrink + lora_expand calls (as raw bits).
    folded=True/False: also check whether the combined call summed the K splits inside the
    expand, seen from t (zero-filled by the harness), whose rows of tokens in segments of 64
    or more are then left unwritten."""
    out = []
    for fused in (True, False):
        dw = DeviceWorkload(wl, y_dtype=y_dtype, **kw)
        dw.build_segments()
        if fused:
            dw.sgmv()
        else:
            dw.shrink()
            dw.expand()
        torch.cuda.synchronize()
        out.append([from_device(dw.y_of(m)).copy() for m in range(wl.n_modules)])
        if fused and folded is not None:
            ids = np.asarray(wl.ids)
            valid = ids[(ids >= 0) & (ids < wl.n_slots)]
            counts = np.bincount(valid, minlength=wl.n_slots)
            long_rows = np.nonzero((ids >= 0) & (ids < wl.n_slots) & (counts[np.clip(ids, 0, None)] >= 64))[0]
            t = dw.t.cpu().numpy()
            untouched = not np.any(t[:, long_rows, :])
            assert untouched == folded, f"partial tiles summed in the expand: {untouched}, expected {folded}"
        dw.close()
    return out


def _calls_with_split(wl, ks):
    """y after lora_shrink per x run, each given a workspace that holds exactly ks K splits of
    its modules (lora_shrink_workspace_bytes covers 8), then lora_expand."""
    dw = DeviceWorkload(wl)
    dw.build_segments()
    n = len(wl.ids)
    per_split = sgr.lora_shrink_workspace_bytes(dw.pool, n, 1) // 8   # one split of one module
    for (m0, m1) in dw.in_groups:
        h_in = wl.modules[m0].h_in
        for (a, b, xo, msx) in dw._x_runs(m0, m1):
            sgr.lora_shrink(dw.pool, a, b - a, dw._xp(xo), h_in, msx, dw.seg, dw.t[a], dw.ld_t, dw.t.stride(0),
                            dw.ws, per_split * ks * (b - a))
    dw.expand()
    torch.cuda.synchronize()
    out = [from_device(dw.y_of(m)).copy() for m in range(wl.n_modules)]
    dw.close()
    return out


def _assert_same_bits(a, b, what):
    for m, (ya, yb) in enumerate(zip(a, b)):
        assert ya.dtype == yb.dtype
        assert np.array_equal(ya.view(np.uint8), yb.view(np.uint8)), f"{what}: module {m}"


@pytest.mark.parametrize("name", ["c3", "c4"])
def test_full_size_same_bits_as_two_calls(name):
    """The mixed-rank batch (17 tiles, rank cap 64; lora_apply_sgmv: K split 8 ways, as
    lora_shrink splits it) and a prefill of 4096 tokens on q, k, v sharing x beside o
    (lora_apply_sgmv_multi: both runs' tiles in one shrink launch, each run aiming at half
    of lora_shrink's workgroups, so 64 tiles split K 4 ways; one partial layout, one expand
    over the four modules), against lora_shrink + lora_expand with the same split."""
    wl = (W.c3_sgmv_prefill if name == "c3" else W.c4_mixed_rank)(draw_w=False)
    say(f"{name}: lora_apply_sgmv vs lora_shrink + lora_expand")
    if name == "c4":
        fused, calls = _both(wl, folded=True)
    else:
        fused, _ = _both(wl, folded=True)
        calls = _calls_with_split(wl, 4)
    _assert_same_bits(fused, calls, name)


def test_c4_fp32_output_same_bits():
    wl = W.c4_mixed_rank(draw_w=False)
    fused, calls = _both(wl, y_dtype="f32")
    _assert_same_bits(fused, calls, "c4 fp32 y")


@pytest.mark.parametrize("rank", [32, 48, 64])
def test_shared_x_rank_caps_same_bits_and_oracle(rank):
    """q, k, v share x at h = 4096 on pools of rank cap 32, 48 and 64: partial tile
    rows of 2, 3 and 4 column groups per thread, K split across workgroups."""
    wl = W.c3_sgmv_prefill(h=4096, rank=rank, units=(2, 8), total_units=32)
    say(f"shared x, rank {rank}, lengths {wl.notes['segment_lengths'].tolist()}")
    fused, calls = _both(wl, folded=True)
    _assert_same_bits(fused, calls, f"rank {rank}")
    for m in range(wl.n_modules):
        assert_close(lo.decode(fused[m], "bf16"), lo.apply_to_y0(wl, m), "bf16", f"rank {rank} m{m}")


@pytest.mark.parametrize("n_modules", [12, 33])
def test_many_modules_own_x_same_bits(n_modules):
    """Modules with their own x in one call (no shared x): one K split per module group."""
    wl = W.c2_bgmv_decode(n_modules=n_modules, h=512, n_tokens=300)
    wl.ids = wl.ids.copy()
    wl.ids[:200] = 3                 # a long segment next to the decode tokens
    fused, calls = _both(wl)
    _assert_same_bits(fused, calls, f"{n_modules} modules")
    for m in (0, n_modules - 1):
        assert_close(lo.decode(fused[m], "bf16"), lo.apply_to_y0(wl, m), "bf16", f"{n_modules} modules m{m}")


def test_fp32_pool_and_no_workspace():
    """fp32 pools take the GEMV path only (no split); without a workspace nothing splits."""
    wl = W.c1_tiny_f32()
    fused, calls = _both(wl)
    _assert_same_bits(fused, calls, "c1 f32")
    wl = W.c4_mixed_rank(draw_w=False)
    dw = DeviceWorkload(wl)
    dw.build_segments()
    sgr.lora_apply_sgmv(dw.pool, 0, 1, dw._xp(0), 4096, 0, dw.seg, dw.t[0], dw.ld_t, dw.t.stride(0), dw.y_of(0), 4096,
                        dw.y[0].stride(0), sgr.LORA_BF16, None, 0)
    torch.cuda.synchronize()
    got = lo.decode(from_device(dw.y_of(0)), "bf16")
    assert_close(got, lo.apply_to_y0(wl, 0), "bf16", "c4 without workspace")
    dw.close()


def test_run_twice_same_bits():
    wl = W.c4_mixed_rank(draw_w=False)
    dw = DeviceWorkload(wl)
    res = []
    for _ in range(2):
        dw.reset_y()
        dw.sgmv_step()
        torch.cuda.synchronize()
        res.append(from_device(dw.y_of(0)).copy())
    assert np.array_equal(res[0], res[1])
    dw.close()


def test_argument_errors_launch_nothing():
    wl = W.c4_mixed_rank(draw_w=False)
    dw = DeviceWorkload(wl)
    dw.build_segments()
    torch.cuda.synchronize()
    y_before = dw.y_of(0).clone()
    base = dict(x=dw._xp(0), ld_x=4096, t=dw.t[0], ld_t=dw.ld_t, y=dw.y_of(0), ld_y=4096, ws=dw.ws.data_ptr(),
                ws_bytes=dw.ws_bytes, ydtype=sgr.LORA_BF16)
    cases = [
        (dict(ws=dw.ws.data_ptr() + 8), -1),          # workspace not 16-byte aligned
        (dict(ld_y=4000), -1),                         # y rows shorter than h_out
        (dict(t=dw.t[0].data_ptr() + 4), -1),          # t not 16-byte aligned
        (dict(ydtype=7), -6),                          # unknown y dtype
    ]
    for kw, code in cases:
        a = dict(base)
        a.update(kw)
        with pytest.raises(sgr.LoraError) as ei:
            sgr.lora_apply_sgmv(dw.pool, 0, 1, a["x"], a["ld_x"], 0, dw.seg, a["t"], a["ld_t"], dw.t.stride(0), a["y"],
                                a["ld_y"], dw.y[0].stride(0), a["ydtype"], a["ws"], a["ws_bytes"])
        assert ei.value.status == code, kw
    torch.cuda.synchronize()
    assert torch.equal(y_before.view(torch.int16), dw.y_of(0).view(torch.int16))
    dw.close()


def test_multi_runs_must_cover_the_modules():
    wl = W.c3_sgmv_prefill(h=4096, rank=16, units=(2, 8), total_units=32)
    dw = DeviceWorkload(wl)
    dw.build_segments()
    torch.cuda.synchronize()
    y = dw.y[0]
    qkv = (dw._xp(dw.x_off[0]), 4096, 0, 3)
    o = (dw._xp(dw.x_off[1]), 4096, 0, 1)
    for runs in ([qkv], [qkv, o, o], [(qkv[0], 4096, 0, 0), qkv, o], []):
        with pytest.raises(sgr.LoraError) as ei:
            sgr.lora_apply_sgmv_multi(dw.pool, 0, 4, runs, dw.seg, dw.t[0], dw.ld_t, dw.t.stride(0), y, 4096,
                                      y.stride(0), sgr.LORA_BF16, dw.ws, dw.ws_bytes)
        assert ei.value.status == -1, len(runs)
    dw.close()

