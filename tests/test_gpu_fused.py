"""GPU parity of lora_fused_gemm (base product and adapter term in one pass)
against the fp64 oracle: y_i = x_i W + s_a (x_i A_a^T) B_a.

Two bars:
* y itself: the bf16 parity bar (rel-L2 <= 5e-3, max-abs <= 2e-2 max|y|);
* the adapter term alone, y - x W against the oracle's term: y is rounded to
  bf16 once, which moves each element by at most half a unit in the last
  place (2^-8 relative), so the term's error has an rms of at most
  rms(y) 2^-8 / sqrt(3); the bound is twice that over rms(term), plus 1e-3
  for the fp32 sums.  A wrong or missing term fails it even where W
  dominates y.
"""
import numpy as np
import pytest

import workloads as W
from oracle import lora_oracle as lo

from gpu_util import assert_close, rel_l2, say

pytestmark = pytest.mark.gpu


def _term_bound(y, term):
    noise = np.sqrt(np.mean(y ** 2)) * 2.0 ** -8 / np.sqrt(3.0)
    return 2.0 * noise / max(np.sqrt(np.mean(term ** 2)), 1e-300) + 1e-3


def _check(dw, m, tokens=None, what=""):
    from segmented_gathered_rank_amd.harness import from_device
    wl = dw.wl
    toks = list(range(wl.n_tokens)) if tokens is None else list(tokens)
    y = lo.decode(from_device(dw.y_of(m)), "bf16")[np.asarray(toks)]
    base = lo.base_product(wl, m, toks)
    term = lo.lora_delta(wl, m, toks)
    assert_close(y, base + term, "bf16", f"{what} module {m} y")
    r = rel_l2(y - base, term)
    lim = _term_bound(y, term)
    assert r <= lim, f"{what} module {m} adapter term: rel-L2 {r:.3e} > {lim:.3e}"
    return r


def _sample(wl, k, seed):
    """Token sample: both ends of every 256-token tile, plus k random tokens."""
    n = wl.n_tokens
    rng = np.random.default_rng(seed)
    s = set()
    for t0 in range(0, n, 256):
        s.update([t0, min(n, t0 + 256) - 1])
    s.update(rng.integers(0, n, size=k).tolist())
    return sorted(s)


def test_fused_small_mixed_every_token():
    """Ragged token and column tiles, ranks 1..64 (up to four 16-row units per
    adapter, so several passes over K), runs, id -1, out-of-range ids and a
    decode-like stretch; every token against the oracle."""
    from segmented_gathered_rank_amd.harness import DeviceWorkload
    import torch
    wl = W.fused_tiles()
    say("fused_tiles: n=600 h_in=320 h_out=384 page=64 ranks 1..64")
    dw = DeviceWorkload(wl)
    dw.fused()
    torch.cuda.synchronize()
    r = _check(dw, 0, what="fused_tiles")
    say(f"  adapter term rel-L2 {r:.2e}")
    # deterministic: a second call writes the same bits
    y1 = dw.y_of(0).clone()
    dw.fused()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), dw.y_of(0).view(torch.int16))
    dw.close()


def test_fused_base_only():
    """ids = NULL: y = x W alone, against the oracle's base product."""
    from segmented_gathered_rank_amd.harness import DeviceWorkload, from_device
    import torch
    wl = W.fused_tiles(seed=15)
    say("fused_tiles base only")
    dw = DeviceWorkload(wl)
    dw.fused(adapters=False)
    torch.cuda.synchronize()
    y = lo.decode(from_device(dw.y_of(0)), "bf16")
    assert_close(y, lo.base_product(wl, 0), "bf16", "base only")
    dw.close()


def test_fused_single_token_and_one_tile():
    """Batches of 1 and 37 tokens (one partial tile) with page size 64."""
    from segmented_gathered_rank_amd.harness import DeviceWorkload
    import torch
    for n in (1, 37):
        wl = W.fused_tiles(seed=16 + n, decode_tokens=0)
        wl.ids = wl.ids[-n:].copy() if n == 37 else wl.ids[:1].copy()
        wl.x = [x[:n].copy() for x in wl.x]
        wl.y0 = [y[:n].copy() for y in wl.y0]
        say(f"fused n={n}")
        dw = DeviceWorkload(wl)
        dw.fused()
        torch.cuda.synchronize()
        _check(dw, 0, what=f"n={n}")
        dw.close()


def test_fused_c3_prefill_sampled():
    """Full-size q, k, v, o of 4096 x 4096 over 4096 prefill tokens in 8
    segments; sampled tokens of every module against the oracle."""
    from segmented_gathered_rank_amd.harness import DeviceWorkload
    import torch
    wl = W.c3_sgmv_prefill()
    say("c3 fused: 4096 tokens, 4 x 4096^2")
    dw = DeviceWorkload(wl)
    dw.fused()
    torch.cuda.synchronize()
    toks = _sample(wl, 24, 3)
    for m in range(wl.n_modules):
        _check(dw, m, toks, what="c3")
    dw.close()


def test_fused_c5_encoder_sampled():
    """Full-size encoder step (qkv, o, up, down) over 32768 tokens with 1,024
    adapters; sampled tokens of every module against the oracle."""
    from segmented_gathered_rank_amd.harness import DeviceWorkload
    import torch
    wl = W.c5_encoder_step()
    say("c5 fused: 32768 tokens, qkv/o/up/down")
    dw = DeviceWorkload(wl)
    dw.fused()
    torch.cuda.synchronize()
    toks = _sample(wl, 16, 5)
    for m in range(wl.n_modules):
        _check(dw, m, toks, what="c5")
    dw.close()


def test_fused_argument_errors():
    import torch
    import segmented_gathered_rank_amd as sgr
    from segmented_gathered_rank_amd.harness import DeviceWorkload
    wl = W.fused_tiles(seed=19)
    dw = DeviceWorkload(wl)
    dw.upload_weights()
    x = dw._xp(0)
    y = dw.y_of(0)
    cases = [
        (dict(ld_x=100), -1),        # leading dimension below h_in
        (dict(ld_y=100), -1),
        (dict(module=1), -1),        # no such module
        (dict(n=-1), -1),
        (dict(x=x + 2), -1),         # rows not 16-byte aligned
    ]
    for kw, code in cases:
        args = dict(module=0, x=x, ld_x=320, w=dw.wT[0], ld_w=320, ids=dw.ids, n=wl.n_tokens, y=y, ld_y=384)
        args.update(kw)
        with pytest.raises(sgr.LoraError) as ei:
            sgr.lora_fused_gemm(dw.pool, args["module"], args["x"], args["ld_x"], args["w"], args["ld_w"],
                                args["ids"], args["n"], args["y"], args["ld_y"])
        assert ei.value.status == code, kw
    # n = 0: nothing to do, nothing written
    before = y.clone()
    sgr.lora_fused_gemm(dw.pool, 0, x, 320, dw.wT[0], 320, dw.ids, 0, y, 384)
    torch.cuda.synchronize()
    assert torch.equal(before.view(torch.int16), y.view(torch.int16))
    dw.close()
    # fp32 pools are refused
    wl1 = W.c1_tiny_f32()
    dw1 = DeviceWorkload(wl1)
    with pytest.raises(sgr.LoraError) as ei:
        sgr.lora_fused_gemm(dw1.pool, 0, dw1._xp(0), 64, dw1._xp(0), 64, dw1.ids, 16, dw1.y_of(0), 64)
    assert ei.value.status == -6
    dw1.close()


def test_fused_rejects_rows_of_too_many_pages():
    """h_in / page_elems above 32 (A page ids per rank row held in LDS): SHAPE, nothing launched."""
    import torch
    import segmented_gathered_rank_amd as sgr
    pool = sgr.lora_pool_create(0, sgr.LORA_BF16, 64, 64, 2, 1, [64 * 33], [64], 4)
    x = torch.zeros(4, 64 * 33, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(64, 64 * 33, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda")
    ids = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(sgr.LoraError) as ei:
        sgr.lora_fused_gemm(pool, 0, x, 64 * 33, w, 64 * 33, ids, 4, y, 64)
    assert ei.value.status == -2
    sgr.lora_pool_destroy(pool)
