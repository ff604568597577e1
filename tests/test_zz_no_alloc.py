"""lora_shrink_noalloc: the shrink for callers that cannot allocate (GPU; C ABI).

Its K-split partial tiles live in a device array that the library holds, so
the call takes no workspace.  It makes the split lora_shrink makes with a full
workspace, so t must match lora_shrink's bit for bit.  Two calls in a row, the
second with a smaller batch (the array keeps the first call's contents), then
a call whose split would need more than the array holds.
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
from segmented_gathered_rank_amd.harness import DeviceWorkload  # noqa: E402


def _shrink_both(dw):
    """t from lora_shrink (full workspace) and from lora_shrink_noalloc, same inputs,
    both buffers first filled with the same garbage."""
    mods = dw.wl.modules
    t_ref = torch.full_like(dw.t, float("nan"))
    t_na = torch.full_like(dw.t, float("nan"))
    ws_bytes = max(sgr.lora_shrink_workspace_bytes(dw.pool, dw.n, len(mods)), 16)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dw.dev)
    dw.build_segments()
    for (m0, m1) in dw.in_groups:
        h_in = mods[m0].h_in
        for (a, b, xo, msx) in dw._x_runs(m0, m1):
            sgr.lora_shrink(dw.pool, a, b - a, dw._xp(xo), h_in, msx, dw.seg, t_ref[a], dw.ld_t,
                            t_ref.stride(0), ws, ws_bytes)
            sgr.lora_shrink_noalloc(dw.pool, a, b - a, dw._xp(xo), h_in, msx, dw.seg, t_na[a], dw.ld_t,
                                    t_na.stride(0))
    torch.cuda.synchronize()
    return t_ref.cpu().numpy(), t_na.cpu().numpy()


def _check_against_oracle(wl, t, tokens):
    """Sampled rows against the oracle's t (fp32 accumulation bar)."""
    for m in range(wl.n_modules):
        ref = lo.shrink_t(wl, m, tokens)
        got = t[m][np.asarray(tokens)][:, :ref.shape[1]]
        mask = ~np.isnan(ref)
        err = np.linalg.norm(got[mask] - ref[mask]) / max(np.linalg.norm(ref[mask]), 1e-300)
        assert err <= 1e-5, (m, err)


def test_noalloc_shrink_matches_lora_shrink_twice_then_rejects():
    # first call: the q,k,v + o prefill, whose q,k,v split fills 12 MiB of the array
    wl = W.c3_sgmv_prefill(draw_w=False)
    dw = DeviceWorkload(wl, device=0)
    say("noalloc: prefill 4096 tokens, q,k,v shared x + o")
    t_ref, t_na = _shrink_both(dw)
    assert np.array_equal(t_ref, t_na, equal_nan=True)
    _check_against_oracle(wl, t_na, list(range(0, wl.n_tokens, 97)))
    dw.close()

    # second call, smaller: the mixed-rank batch (ranks up to 64, decode tokens and prefill segments)
    wl2 = W.c4_mixed_rank(draw_w=False)
    dw2 = DeviceWorkload(wl2, device=0)
    say("noalloc: mixed-rank batch 1072 tokens")
    t_ref, t_na = _shrink_both(dw2)
    assert np.array_equal(t_ref, t_na, equal_nan=True)
    _check_against_oracle(wl2, t_na, list(range(0, wl2.n_tokens, 7)))
    dw2.close()

    # a split that needs more than the array: two rank-64 modules of 4096 sharing x over
    # 4096 tokens take 8 splits of 64 x 64 partial tiles for 128 tiles and 2 modules (32 MiB)
    dev = torch.device("cuda", 0)
    n = 4096
    pool = sgr.lora_pool_create(0, sgr.LORA_BF16, 4096, 4, 8, 2, [4096, 4096], [4096, 4096], 64)
    try:
        buf = torch.zeros(sgr.lora_segments_bytes(n, 8), dtype=torch.uint8, device=dev)
        seg = sgr.lora_segments_bind(buf, n, 8)
        x = torch.zeros(n, 4096, dtype=torch.bfloat16, device=dev)
        t = torch.zeros(2, n, 64, dtype=torch.float32, device=dev)
        need = 128 * 2 * 8 * 64 * 64 * 4
        assert need > sgr.LORA_NOALLOC_SCRATCH_BYTES
        with pytest.raises(sgr.LoraError) as err:
            sgr.lora_shrink_noalloc(pool, 0, 2, x, 4096, 0, seg, t, 64, t.stride(0))
        assert err.value.status == -9   # LORA_ERR_WORKSPACE, nothing launched
        torch.cuda.synchronize()
    finally:
        sgr.lora_pool_destroy(pool)
