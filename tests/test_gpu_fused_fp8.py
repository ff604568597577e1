"""GPU parity of lora_fused_gemm_fp8w (FP8 base, bf16 adapters) against the
fp64 oracle: y_i = w_scale * x_i E(W8) + s_a (x_i A_a^T) B_a, E the exact
value of an OCP E4M3 code.

Widening an E4M3 code to bf16 is exact, so the kernel's products are exact
and only fp32 summation and the one bf16 rounding of y remain: the bars are
those of the bf16 fused pass (y itself, and the adapter term alone), and the
code sweep is compared bit for bit.
"""
import numpy as np
import pytest

import workloads as W
from oracle import lora_oracle as lo

from gpu_util import assert_close, rel_l2, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import segmented_gathered_rank_amd as sgr  # noqa: E402
from segmented_gathered_rank_amd.harness import DeviceWorkload, from_device  # noqa: E402


def _term_bound(y, term):
    noise = np.sqrt(np.mean(y ** 2)) * 2.0 ** -8 / np.sqrt(3.0)
    return 2.0 * noise / max(np.sqrt(np.mean(term ** 2)), 1e-300) + 1e-3


def _check(dw, m, tokens=None, what=""):
    wl = dw.wl
    toks = list(range(wl.n_tokens)) if tokens is None else list(tokens)
    y = lo.decode(from_device(dw.y_of(m)), "bf16")[np.asarray(toks)]
    base = lo.base_product_fp8w(wl, m, toks)
    term = lo.lora_delta(wl, m, toks)
    assert_close(y, base + term, "bf16", f"{what} module {m} y")
    r = rel_l2(y - base, term)
    lim = _term_bound(y, term)
    assert r <= lim, f"{what} module {m} adapter term: rel-L2 {r:.3e} > {lim:.3e}"
    return r


def _sample(wl, k, seed):
    n = wl.n_tokens
    rng = np.random.default_rng(seed)
    s = set()
    for t0 in range(0, n, 256):
        s.update([t0, min(n, t0 + 256) - 1])
    s.update(rng.integers(0, n, size=k).tolist())
    return sorted(s)


@pytest.mark.parametrize("adapters", [False, True])
def test_fp8w_every_code_bit_exact(adapters):
    """x = identity, W8[k][c] = (k + c) mod 256, scale 1: y[i][c] is the value
    of one code, which bf16 holds exactly; all 254 finite codes, bit for bit."""
    wl = W.fp8_code_sweep()
    say(f"fp8 code sweep (adapters={adapters})")
    dw = DeviceWorkload(wl, extra_pages=4)
    dw.fused_fp8(adapters=adapters)
    torch.cuda.synchronize()
    y = lo.decode(from_device(dw.y_of(0)), "bf16")
    ref = lo.base_product_fp8w(wl, 0)
    assert np.array_equal(y, ref)
    assert np.array_equal(np.signbit(y), np.signbit(ref))    # -0 stays -0
    dw.close()


def test_fp8w_nan_code_poisons_its_column():
    """The NaN codes (0x7F, 0xFF): every output of a column whose weights hold
    one is NaN (0 x NaN is NaN), as in the fp64 definition; other columns exact."""
    wl = W.fp8_code_sweep(nan_codes=True)
    dw = DeviceWorkload(wl, extra_pages=4)
    dw.fused_fp8(adapters=False)
    torch.cuda.synchronize()
    y = lo.decode(from_device(dw.y_of(0)), "bf16")
    ref = lo.base_product_fp8w(wl, 0)
    assert np.array_equal(np.isnan(y), np.isnan(ref))
    assert np.isnan(ref).any()
    fin = ~np.isnan(ref)
    assert np.array_equal(y[fin], ref[fin])
    dw.close()


def test_fp8w_small_mixed_every_token():
    """The fused-pass tile workload (ragged tiles, ranks 1..64, id -1, out-of-range
    ids) with its base quantized to E4M3 per output column; every token."""
    wl = W.with_fp8_base(W.fused_tiles())
    say("fused_tiles fp8 base: n=600 h_in=320 h_out=384")
    dw = DeviceWorkload(wl)
    dw.fused_fp8()
    torch.cuda.synchronize()
    r = _check(dw, 0, what="fused_tiles fp8")
    say(f"  adapter term rel-L2 {r:.2e}")
    y1 = dw.y_of(0).clone()
    dw.fused_fp8()
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), dw.y_of(0).view(torch.int16))
    dw.close()


def test_fp8w_base_only():
    wl = W.with_fp8_base(W.fused_tiles(seed=15))
    dw = DeviceWorkload(wl)
    dw.fused_fp8(adapters=False)
    torch.cuda.synchronize()
    y = lo.decode(from_device(dw.y_of(0)), "bf16")
    assert_close(y, lo.base_product_fp8w(wl, 0), "bf16", "fp8 base only")
    dw.close()


@pytest.mark.parametrize("name", ["c3", "c5"])
def test_fp8w_full_size_sampled(name):
    """Full-size q,k,v,o of 4096^2 over 4096 prefill tokens, and the encoder layer
    over 32768 tokens with 1,024 adapters: sampled tokens of every module."""
    wl = W.with_fp8_base(W.c3_sgmv_prefill() if name == "c3" else W.c5_encoder_step())
    say(f"{name} fused fp8 base: {wl.n_tokens} tokens")
    dw = DeviceWorkload(wl)
    dw.fused_fp8()
    torch.cuda.synchronize()
    toks = _sample(wl, 16, 3 if name == "c3" else 5)
    for m in range(wl.n_modules):
        _check(dw, m, toks, what=f"{name} fp8")
    dw.close()


def test_fp8w_argument_errors():
    wl = W.with_fp8_base(W.fused_tiles(seed=19))
    dw = DeviceWorkload(wl)
    dw.upload_weights_fp8()
    x, y = dw._xp(0), dw.y_of(0)
    w8, sc = dw.w8T[0], dw.w8s[0]
    cases = [
        (dict(w8=w8.data_ptr() + 8), -1),     # codes not 16-byte aligned
        (dict(ld_w=328), -1),                 # row stride not a multiple of 16
        (dict(ld_w=304), -1),                 # below h_in
        (dict(sc=None), -1),                  # no scales
        (dict(sc=sc.data_ptr() + 4), -1),     # scales not 16-byte aligned
        (dict(module=1), -1),
    ]
    for kw, code in cases:
        args = dict(module=0, w8=w8, ld_w=320, sc=sc)
        args.update(kw)
        with pytest.raises(sgr.LoraError) as ei:
            sgr.lora_fused_gemm_fp8w(dw.pool, args["module"], x, 320, args["w8"], args["ld_w"], args["sc"],
                                     dw.ids, wl.n_tokens, y, 384)
        assert ei.value.status == code, kw
    dw.close()
