"""Pins of the CPU oracle against facts outside itself (CPU only).

Each pin cites where its fact comes from:
* the worked example of the study page "Multi-LoRA Serving" (section "The
  kernel trick: gather, do not merge"): its printed outputs are stored in
  tests/golden/worked_example.json;
* the merged-weight identity W' = W + AB (slide 5 of "Thousands of
  adapters"; option 1 of the study page's demo);
* closed forms (rank-1 fingerprints, scale 0, id -1, linearity in B);
* exact rational brute force on tiny inputs.

The last block plants plausible mistakes in the oracle (on the CPU) and
checks that at least one pin catches each of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import lora_oracle as lo
import workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


# ---------------------------------------------------------------- helpers
def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _small_bf16():
    return W.c2_bgmv_decode(seed=7, n_tokens=24, h=256, n_slots=5, rank=8)


def _with_adapters(wl, fn):
    """Copy of ``wl`` with every adapter tuple replaced by fn(rank, scale, A, B)."""
    import copy
    w2 = copy.copy(wl)
    w2.adapters = [[None if a is None else fn(*a) for a in row] for row in wl.adapters]
    return w2


def pin_merged(o=lo):
    """P1: gathered form == merged-weight form (fp64) on fp32 and bf16 inputs."""
    ok = True
    for wl in (W.c1_tiny_f32(), _small_bf16()):
        for m in range(wl.n_modules):
            ok &= _rel(o.lora_forward(wl, m), o.merged_forward(wl, m)) <= 1e-12
    return ok


def pin_worked_example(o=lo):
    """P13: the page's demo.  Its batch holds 34 distinct adapters, and the page
    reports the merged-weight and gathered outputs equal within 1e-3.  Checked:
    the oracle's gathered form against the same sum written in the page's own
    operand layout (W x + s B (A x) per token, fp64, so the layout mapping of the
    workload is checked too), and the oracle's merged form against its gathered
    form at the page's tolerance."""
    gold = json.load(open(GOLD))["printed"]
    wl = W.c0_worked_example()
    if len(np.unique(wl.ids)) != gold["distinct_adapters_in_batch"]:
        return False
    Wp, Ap, Bp = (wl.notes[k].astype(np.float64) for k in ("W_page", "A_page", "B_page"))
    X = wl.x[0].astype(np.float64)
    low = np.einsum("nrd,nd->nr", Ap[wl.ids], X)                 # A_a x_i, page layout
    page_form = X @ Wp.T + 2.0 * np.einsum("ndr,nr->nd", Bp[wl.ids], low)
    gathered = o.lora_forward(wl, 0)
    if _rel(gathered, page_form) > 1e-12:
        return False
    same = bool(np.allclose(o.merged_forward(wl, 0), gathered, atol=1e-3))
    return same == gold["same_outputs_allclose_atol_1e-3"]


def pin_fingerprint(o=lo):
    """P4: rank-1 one-hot adapters: the term is x_i[j_a] in column k_a only."""
    wl = W.fingerprint_rank1(dtype="f32")
    d = o.lora_delta(wl, 0)
    x = o.decode(wl.x[0], "f32")
    exp = np.zeros_like(d)
    for i, a in enumerate(wl.ids):
        if 0 <= a < wl.n_slots:
            exp[i, wl.notes["k"][a]] = x[i, wl.notes["j"][a]]
    return bool(np.array_equal(d, exp))


def _frac_forward(x, Wm, A, B, scale, ids):
    """Exact rational y_i = x_i W + s (x_i A_a^T) B_a, by triple loops."""
    n, h_in = len(x), len(x[0])
    h_out = len(Wm[0])
    out = []
    for i in range(n):
        row = []
        a = ids[i]
        for c in range(h_out):
            acc = Fraction(0)
            for k in range(h_in):
                acc += Fraction(float(x[i][k])) * Fraction(float(Wm[k][c]))
            if a >= 0:
                for j in range(len(A[a])):
                    tj = Fraction(0)
                    for k in range(h_in):
                        tj += Fraction(float(x[i][k])) * Fraction(float(A[a][j][k]))
                    acc += Fraction(float(scale[a])) * tj * Fraction(float(B[a][j][c]))
            row.append(acc)
        out.append(row)
    return out


def _tiny(seed, integer):
    rng = np.random.default_rng(seed)
    n, h_in, h_out, n_slots = 6, 8, 5, 3

    def draw(shape):
        if integer:
            return rng.integers(-4, 5, shape).astype(np.float32)
        return rng.normal(0, 1, shape).astype(np.float32)

    ranks = [1, 2, 2]
    wl = W.Workload(
        "tiny", "f32", 1, n_slots, [W.Module("p", h_in, h_out, 0)],
        np.array([0, 2, -1, 1, 0, 2], np.int32), [draw((n, h_in))],
        [np.zeros((n, h_out), np.float32)], [draw((h_in, h_out))],
        [[(ranks[s], 2.0 if integer else 0.75, draw((ranks[s], h_in)),
           draw((ranks[s], h_out)))] for s in range(n_slots)])
    return wl


def pin_bruteforce(o=lo):
    """P5/P6: exact rationals.  Integer inputs: bit-exact.  Random fp32 inputs:
    within fp64 rounding (1e-13 relative per element)."""
    ok = True
    for seed, integer in ((1, True), (2, False), (3, False)):
        wl = _tiny(seed, integer)
        A = [a[2] for a in (row[0] for row in wl.adapters)]
        B = [a[3] for a in (row[0] for row in wl.adapters)]
        sc = [a[1] for a in (row[0] for row in wl.adapters)]
        exact = _frac_forward(wl.x[0], wl.W[0], A, B, sc, wl.ids)
        got = o.lora_forward(wl, 0)
        ex = np.array([[float(v) for v in r] for r in exact])
        if integer:
            ok &= bool(np.array_equal(got, ex))
        else:
            ok &= bool(np.all(np.abs(got - ex) <= 1e-13 * np.maximum(1.0, np.abs(ex))))
    return ok


def pin_scale_zero(o=lo):
    """P14: scale 0 leaves y = x W exactly."""
    wl = _with_adapters(W.c1_tiny_f32(), lambda r, s, A, B: (r, 0.0, A, B))
    return bool(np.array_equal(o.lora_forward(wl, 0), o.base_product(wl, 0)))


def pin_no_adapter(o=lo):
    """P2: id -1 (and ids out of range) give y = x W bit for bit, and no term."""
    wl = W.c1_tiny_f32()
    wl.ids = wl.ids.copy()
    wl.ids[0] = 99            # out of range: treated as -1
    neg = np.nonzero((wl.ids < 0) | (wl.ids >= wl.n_slots))[0]
    if neg.size == 0:
        return False
    y = o.lora_forward(wl, 0, neg)
    return bool(np.array_equal(y, o.base_product(wl, 0, neg))
                and not np.any(o.lora_delta(wl, 0, neg)))


def pin_linearity(o=lo):
    """P3: delta(B1 + 2 B2) = delta(B1) + 2 delta(B2) (B values on a 1/64 grid, so
    B1 + 2 B2 is exact in fp32)."""
    rng = np.random.default_rng(5)
    base = W.c1_tiny_f32()
    grid = lambda shp: (rng.integers(-64, 65, shp) / 64.0).astype(np.float32)
    B1 = [grid(a[3].shape) for row in base.adapters for a in row]
    B2 = [grid(a[3].shape) for row in base.adapters for a in row]
    it1, it2, it3 = iter(B1), iter(B2), iter([b1 + 2 * b2 for b1, b2 in zip(B1, B2)])
    w1 = _with_adapters(base, lambda r, s, A, B: (r, s, A, next(it1)))
    w2 = _with_adapters(base, lambda r, s, A, B: (r, s, A, next(it2)))
    w3 = _with_adapters(base, lambda r, s, A, B: (r, s, A, next(it3)))
    d1, d2, d3 = o.lora_delta(w1, 0), o.lora_delta(w2, 0), o.lora_delta(w3, 0)
    return _rel(d3, d1 + 2 * d2) <= 1e-12


def pin_shrink_columns(o=lo):
    """P15: t's column j is rank row j's dot product with x (ranks 2..5, integer
    inputs, so the exact sums are Python integers); columns past the rank and
    tokens without an adapter are NaN."""
    wl = W.integer_exact(seed=31, n_tokens=40, ranks=[2, 3, 4, 5, 2, 3])
    t = o.shrink_t(wl, 0)
    x = wl.x[0].astype(np.int64)
    for i, a in enumerate(wl.ids):
        if not 0 <= a < wl.n_slots:
            if not np.all(np.isnan(t[i])):
                return False
            continue
        rank, _, A, _ = wl.adapters[a][0]
        want = [sum(int(p) * int(q) for p, q in zip(x[i], A[j].astype(np.int64))) for j in range(rank)]
        if t[i, :rank].tolist() != want or not np.all(np.isnan(t[i, rank:])):
            return False
    return True


ALL_PINS = [pin_merged, pin_worked_example, pin_fingerprint, pin_bruteforce,
            pin_scale_zero, pin_no_adapter, pin_linearity,
            pin_shrink_columns]


# ---------------------------------------------------------------- the pins
@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin_holds(pin):
    assert pin()


def test_worked_example_closed_forms_in_golden():
    """The page prints 2r/d = 1.56% and 0.13 MB vs 8.4 MB for d=2048, r=16, fp16."""
    gold = json.load(open(GOLD))
    d, r = gold["setting"]["d"], gold["setting"]["r"]
    flops_base = 2 * 64 * d * d
    flops_lora = 2 * 64 * r * d * 2
    assert f"{flops_lora / flops_base:.2%}" == gold["printed"]["adapter_flops_overhead_percent"]
    assert f"{2 * r / d:.2%}" == gold["printed"]["two_r_over_d_percent"]
    assert f"{2 * r * d * 2 / 1e6:.2f}" == gold["printed"]["one_adapter_one_layer_MB"]
    assert f"{d * d * 2 / 1e6:.1f}" == gold["printed"]["base_layer_MB"]


def test_apply_to_y0_is_y0_plus_term():
    wl = _small_bf16()
    toks = [0, 3, 7, 23]
    y = lo.apply_to_y0(wl, 0, toks)
    y0 = lo.decode(wl.y0[0][toks], "bf16")
    np.testing.assert_allclose(y - y0, lo.lora_delta(wl, 0, toks), rtol=0, atol=1e-14)


def test_shrink_t_matches_term():
    """t rows reproduce the term when multiplied into B (rank-1 fingerprint: t = x[j])."""
    wl = W.fingerprint_rank1(dtype="f32")
    t = lo.shrink_t(wl, 0)
    x = lo.decode(wl.x[0], "f32")
    for i, a in enumerate(wl.ids):
        if 0 <= a < wl.n_slots:
            assert t[i, 0] == x[i, wl.notes["j"][a]]
        else:
            assert np.isnan(t[i, 0])


# ---------------------------------------------------------------- planted mistakes
def _mutant_no_scale(x_row, A, B, scale):
    t = A @ x_row
    return t @ B, t


def _mutant_sign(x_row, A, B, scale):
    t = A @ x_row
    return -scale * (t @ B), t


def _mutant_rank_order(x_row, A, B, scale):
    t = A @ x_row
    return scale * (t[::-1] @ B), t


def _mutant_last_row_dropped(x_row, A, B, scale):
    t = A[:-1] @ x_row
    return scale * (t @ B[:-1]), t


def _mutant_t_reversed(x_row, A, B, scale):      # right term, t columns in reverse
    t = A @ x_row
    return scale * (t @ B), t[::-1].copy()


def _mutant_t_from_columns(x_row, A, B, scale):  # A read with its strides swapped ([h][r] storage)
    t = A.reshape(A.shape[1], A.shape[0]).T @ x_row
    return scale * ((A @ x_row) @ B), t


def _fails(pin):
    """A pin fails if it returns False or cannot run (a wrongly shaped t raises)."""
    try:
        return not pin()
    except (ValueError, IndexError):
        return True


@pytest.mark.parametrize("mutant", [_mutant_no_scale, _mutant_sign, _mutant_rank_order,
                                    _mutant_last_row_dropped, _mutant_t_reversed,
                                    _mutant_t_from_columns],
                         ids=lambda f: f.__name__)
def test_pins_catch_planted_term_mistakes(monkeypatch, mutant):
    monkeypatch.setattr(lo, "adapter_term", mutant)
    failed = [p.__name__ for p in ALL_PINS if _fails(p)]
    assert failed, "no pin caught the planted mistake"


def test_pins_catch_planted_decode_mistake(monkeypatch):
    real = lo.decode

    def bad_decode(a, dtype):   # bf16 decoded from the wrong half-word
        if dtype == "bf16":
            bits = np.asarray(a, np.uint16).astype(np.uint32) << np.uint32(15)
            return bits.view(np.float32).astype(np.float64)
        return real(a, dtype)

    monkeypatch.setattr(lo, "decode", bad_decode)
    wl = W.c2_bgmv_decode(seed=3, n_tokens=4, h=64, n_slots=2, rank=2)
    # exact decode of a known bf16 pattern: 0x3F80 is 1.0, 0xC000 is -2.0
    assert not np.array_equal(lo.decode(np.array([0x3F80, 0xC000], np.uint16), "bf16"), [1.0, -2.0])
    monkeypatch.setattr(lo, "decode", real)
    assert np.array_equal(lo.decode(np.array([0x3F80, 0xC000], np.uint16), "bf16"), [1.0, -2.0])
    assert wl.n_tokens == 4


# ---------------------------------------------------------------- FP8 base
def _e4m3_pins(decode):
    """The OCP E4M3 decode against what fixes it outside the oracle: a library
    routine over all 256 codes, closed forms and invariants of the format."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    d = decode(codes)
    lib = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ok = np.array_equal(np.isnan(d), np.isnan(lib))
    fin = ~np.isnan(lib)
    ok &= np.array_equal(d[fin], lib[fin]) and np.array_equal(np.signbit(d[fin]), np.signbit(lib[fin]))
    closed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
              0x78: 256.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x80: -0.0}
    for c, v in closed.items():
        ok &= bool(d[c] == v) and bool(np.signbit(d[c]) == np.signbit(v))
    ok &= bool(np.isnan(d[0x7F]) and np.isnan(d[0xFF])) and int(np.isnan(d).sum()) == 2
    pos = d[:0x7F]
    ok &= bool(np.all(np.diff(pos) > 0))                          # magnitudes increase with the code
    ok &= np.array_equal(d[0x80:0xFF], -d[:0x7F])                 # the sign bit only flips the sign
    bf = (np.asarray(pos, np.float32).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    ok &= np.array_equal(bf.astype(np.float64), pos)              # every value is a bf16 value
    return bool(ok)


def test_e4m3_decode_pins():
    assert _e4m3_pins(lo.decode_e4m3)


def test_fp8_base_brute_force_and_identity():
    """base_product_fp8w: exact rationals on a tiny case; the code sweep's identity x."""
    rng = np.random.default_rng(31)
    wl = W.Workload("t8", "bf16", 8, 1, [W.Module("p", 8, 5, 0)], np.array([-1, -1, -1], np.int32),
                    [W.to_bf16_bits(rng.normal(0, 1, (3, 8)).astype(np.float32))],
                    [W.to_bf16_bits(np.zeros((3, 5), np.float32))], [None], [[None]])
    codes = rng.integers(0, 256, (8, 5)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3A
    wl.W8 = [codes]
    wl.W8_scale = [rng.uniform(0.5, 2.0, 5).astype(np.float32)]
    got = lo.base_product_fp8w(wl, 0)
    x = lo.decode(wl.x[0], "bf16")
    val = lo.decode_e4m3(codes)
    for i in range(3):
        for c in range(5):
            exact = sum(Fraction(float(x[i][k])) * Fraction(float(val[k][c])) for k in range(8))
            exact *= Fraction(float(wl.W8_scale[0][c]))
            assert abs(float(exact) - got[i][c]) <= 1e-13 * max(1.0, abs(float(exact)))
    sw = W.fp8_code_sweep()
    y = lo.base_product_fp8w(sw, 0)
    k = np.arange(256)
    codes = ((k[:, None] + k[None, :]) % 256).astype(np.uint8)
    codes[(codes == 0x7F) | (codes == 0xFF)] = 0          # the sweep's stand-in for the NaN codes
    assert np.array_equal(y, lo.decode_e4m3(codes))


def test_e4m3_planted_mistakes_fail_a_pin():
    """A bias of 8 (the other FP8 E4M3 variant), subnormals read as normals, and
    the NaN code read as 480 each fail the decode pins."""
    def bias8(c):
        c = np.asarray(c, np.uint8).astype(np.int64)
        s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
        mag = np.where(e == 0, np.ldexp(m.astype(float), -10), np.ldexp((8 + m).astype(float), e - 11))
        mag = np.where((e == 15) & (m == 7), np.nan, mag)
        return np.where(s == 1, -mag, mag)

    def no_subnormals(c):
        c = np.asarray(c, np.uint8).astype(np.int64)
        s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
        mag = np.ldexp((8 + m).astype(float), e - 10)
        mag = np.where((e == 15) & (m == 7), np.nan, mag)
        return np.where(s == 1, -mag, mag)

    def nan_as_480(c):
        d = lo.decode_e4m3(c)
        return np.where(np.isnan(d), np.where(np.asarray(c) >= 0x80, -480.0, 480.0), d)

    for mutant in (bias8, no_subnormals, nan_as_480):
        assert not _e4m3_pins(mutant), mutant.__name__
