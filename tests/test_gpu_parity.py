"""Parity of the HIP path with the CPU oracle (GPU; calls go through the C ABI).

Integer and index work is compared bit for bit; floating point within the
stated tolerances (rel-L2 <= 5e-3 and max-abs <= 2e-2 max|y| for bf16,
rel-L2 <= 1e-5 for fp32), or bit for bit where the arithmetic is exact.
"""
import ctypes

import numpy as np
import pytest

import workloads as W
from oracle import lora_oracle as lo
from gpu_util import assert_close, rel_l2, run, say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import segmented_gathered_rank_amd as sgr  # noqa: E402
from segmented_gathered_rank_amd.harness import DeviceWorkload, from_device  # noqa: E402


# ----------------------------------------------------------------- segments
def _gpu_segments(ids, n_slots, buf=None):
    """Builds on the GPU into a buffer that starts out as garbage (0xA5 bytes),
    so that any entry the builder fails to write shows up."""
    dev = torch.device("cuda", 0)
    n = len(ids)
    if buf is None:
        buf = torch.full((max(sgr.lora_segments_bytes(n, n_slots), 256),), 0xA5, dtype=torch.uint8, device=dev)
    seg = sgr.lora_segments_bind(buf, n, n_slots)
    t_ids = torch.tensor(np.asarray(ids, np.int32), dtype=torch.int32, device=dev)
    sgr.lora_build_segments(t_ids, seg)
    st, meta = sgr.lora_segments_check(seg)
    words = buf.view(torch.int32).cpu().numpy()

    def arr(ptr, count):
        off = (ptr - buf.data_ptr()) // 4
        return words[off:off + count]
    return st, meta, seg, arr


SEG_CASES = {
    "one": ([3], 8),
    "all_neg": ([-1] * 100, 4),
    "one_id": ([2] * 300, 4),
    "all_distinct": (list(range(63, -1, -1)), 64),
    "last_slot": ([7, 7, -1, 7] * 20, 8),
    "bad_ids": ([0, 5, -2, 1, 100, -1, 1, 3] * 9, 4),
    "c1": (W.c1_tiny_f32().ids, 4),
    "c2": (W.c2_bgmv_decode(draw_w=False, h=64).ids, 32),
    "c4": (W.c4_mixed_rank(h=128, draw_w=False).ids, 64),
    "many_slots": (np.random.default_rng(9).integers(-1, 8192, 20000), 8192),
    "c5_ids": (np.repeat(W.zipf_ids(np.random.default_rng(5), 128, 1024, 1.2), 256), 1024),
    "long_runs": (np.random.default_rng(3).integers(-1, 6, 5000), 6),
    # schedule boundaries of the builder: 512 tokens per histogram row on one
    # workgroup (64 slots -> 16 rows -> 8192 tokens), chunks of >= 1024 above
    "one_group_max": (np.random.default_rng(21).integers(-1, 64, 8192), 64),
    "chunked_ragged": (np.random.default_rng(22).integers(-1, 64, 8193), 64),
    "chunked_bad_ids": (np.random.default_rng(23).integers(-3, 110, 30001), 100),
    "chunked_one_id": ([3] * 50000, 5),
    "chunked_all_neg": ([-1] * 20000, 16),
    "chunked_one_chunk": (np.random.default_rng(24).integers(-1, 8192, 600), 8192),
    "chunked_runs": (np.repeat(np.random.default_rng(25).integers(0, 300, 1024), 128), 300),
    # long segments whose records the whole workgroup writes (one workgroup; chunked), and more
    # long segments than the builder describes at once (each wave writes its own)
    "one_group_many_long": (np.repeat(np.random.default_rng(26).permutation(100), 64 + 5), 100),
    "chunked_many_long": (np.repeat(np.random.default_rng(27).permutation(400), 130), 400),
    "chunked_too_many_long": (np.repeat(np.random.default_rng(28).permutation(1500), 70), 1500),
    # one-workgroup sizes: one wave up to 512 tokens and 256 slots (4 slots per lane), four
    # waves up to 2048 tokens and 1024 slots, sixteen above; each edge from both sides
    "wave_max": (np.random.default_rng(29).integers(-1, 256, 512), 256),
    "wave_long_segments": (np.repeat(np.random.default_rng(30).permutation(8), 64), 8),
    "quad_tokens": (np.random.default_rng(31).integers(-1, 40, 513), 40),
    "quad_slots": (np.random.default_rng(32).integers(-1, 257, 300), 257),
    "quad_max": (np.random.default_rng(33).integers(-1, 1024, 2048), 1024),
    "quad_long_and_short": (np.concatenate([np.repeat([5, 9], 700), np.arange(600) % 50]), 64),
    "sixteen_from": (np.random.default_rng(34).integers(-1, 64, 2049), 64),
    # batches of up to 64 tokens take one wave with a token per lane (k_segments_tiny): one
    # long segment (64 tokens of one id: units and a tile), the same with bad ids, 8,192 slots
    "tiny_long": ([5] * 64, 8),
    "tiny_long_minus": ([5] * 62 + [-1, 9], 8),
    "tiny_max_slots": (np.random.default_rng(35).integers(-1, 8192, 63), 8192),
    "tiny_runs": (np.repeat(np.random.default_rng(36).integers(0, 5, 16), 4), 5),
    # chunked batches in two launches (layout beside the scatter) up to 65,536 chunk counters,
    # in three (k_seg_scan between them) above: 64 chunks x 1,024 slots, then 65
    "place_max": (np.random.default_rng(37).integers(-1, 1024, 65536), 1024),
    "scan_from": (np.random.default_rng(38).integers(-1, 1024, 65537), 1024),
}


def _check_segments(ids, n_slots, st, meta, seg, arr):
    ref = lo.build_segments(ids, n_slots)
    assert st == (-8 if ref["n_bad"] else 0)
    n_seg = meta[sgr.META["n_seg"]]
    assert n_seg == ref["n_seg"]
    assert meta[sgr.META["n_active"]] == ref["n_active"]
    assert meta[sgr.META["max_seg_len"]] == ref["max_seg_len"]
    assert meta[sgr.META["n_bad"]] == ref["n_bad"]
    assert np.array_equal(arr(seg.perm, ref["n_active"]), ref["perm"])
    assert np.array_equal(arr(seg.seg_start, n_seg + 1), ref["seg_start"])
    assert np.array_equal(arr(seg.seg_slot, n_seg), ref["seg_slot"])
    # work lists: every segment covered exactly once, in the library's chunk sizes
    ut, tt, lmin = meta[sgr.META["unit_tokens"]], meta[sgr.META["tile_tokens"]], meta[sgr.META["long_min"]]
    nus, nua, ntl = meta[sgr.META["n_units_short"]], meta[sgr.META["n_units_all"]], meta[sgr.META["n_tiles"]]
    units = arr(seg.units, 2 * nua).reshape(-1, 2)
    tiles = arr(seg.tiles, 2 * ntl).reshape(-1, 2)
    lens = np.diff(ref["seg_start"])
    exp_units, exp_tiles = [], []

    def unit(k, L, u):   # (slot + 65536 * tokens in the unit + 2^24 * [several units], first position)
        return (int(ref["seg_slot"][k]) + 65536 * min(ut, L - u) + (1 << 24) * (L > ut), int(ref["seg_start"][k]) + u)
    for k, L in enumerate(lens):
        if L < lmin:
            exp_units += [unit(k, L, u) for u in range(0, L, ut)]
    short = list(exp_units)
    for k, L in enumerate(lens):
        s0 = ref["seg_start"][k]
        if L >= lmin:
            exp_units += [unit(k, L, u) for u in range(0, L, ut)]
            exp_tiles += [(int(ref["seg_slot"][k]) + 65536 * min(tt, L - u), int(s0 + u)) for u in range(0, L, tt)]
    # the library's order: short-segment units, then long-segment units, each in segment order
    assert nus == len(short)
    assert list(map(tuple, units.tolist())) == exp_units
    assert list(map(tuple, tiles.tolist())) == exp_tiles


@pytest.mark.parametrize("name", sorted(SEG_CASES))
def test_segments_bit_exact(name):
    ids, n_slots = SEG_CASES[name]
    ids = np.asarray(ids, np.int32)
    say(f"segments case {name}: n={len(ids)} n_slots={n_slots} chunks={_chunks(len(ids), n_slots)}")
    _check_segments(ids, n_slots, *_gpu_segments(ids, n_slots))


def _chunks(n, n_slots):
    """The builder's schedule for a batch: 0 = one workgroup, else its chunks
    (lora_segments_bind does no device work, so a stand-in address serves)."""
    seg = sgr.lora_segments()
    assert sgr._lib.lora_segments_bind(256, 1 << 40, n, n_slots, ctypes.byref(seg)) == 0
    return seg.n_chunks


@pytest.mark.parametrize("n,n_slots", [(3000, 40), (40000, 40), (5000, 8192)])
def test_segments_rebuild_same_buffer(n, n_slots):
    """A second batch built into the same buffer (both schedules): nothing of
    the first batch's layout or scratch leaks into the second."""
    rng = np.random.default_rng(n + n_slots)
    a = rng.integers(-1, n_slots, n).astype(np.int32)
    b = np.sort(rng.integers(-1, n_slots // 2, n)).astype(np.int32)
    say(f"segments rebuild n={n} n_slots={n_slots} chunks={_chunks(n, n_slots)}")
    st, meta, seg, arr = _gpu_segments(a, n_slots)
    _check_segments(a, n_slots, st, meta, seg, arr)
    _check_segments(b, n_slots, *_gpu_segments(b, n_slots, buf=seg._buf))


def test_segments_empty_batch_enqueues_nothing():
    st, meta, seg, arr = _gpu_segments([], 4)
    assert st == 0 and meta[sgr.META["n_seg"]] == 0


# ----------------------------------------------------------------- pool
def test_pool_round_trip_and_page_accounting():
    wl = W.c4_mixed_rank(h=256, prefill_len=64, draw_w=False)
    dw = DeviceWorkload(wl, extra_pages=100, max_rank=64)
    h = wl.page_elems
    st = sgr.lora_pool_stats(dw.pool)
    need = wl.pages_needed()
    assert st["n_pages"] == need + 100 and st["free_pages"] == 100
    assert st["loaded_slots"] == wl.n_slots and st["loaded_entries"] == wl.n_slots
    for s in (0, 5, 63):
        rank, scale, A, B = wl.adapters[s][0]
        Ab = np.zeros_like(A)
        Bb = np.zeros_like(B)
        r, sc, pages = sgr.lora_pool_read(dw.pool, s, 0, Ab, Bb, max_pages=256)
        assert r == rank and sc == scale
        assert np.array_equal(Ab, A) and np.array_equal(Bb, B)
        assert len(set(pages[: rank * 2])) == rank * 2        # r pages for A, r for B (h_in = h_out = h)
    # evict returns exactly the slot's pages; a reload may land elsewhere
    r5 = wl.adapters[5][0][0]
    sgr.lora_pool_evict(dw.pool, 5)
    assert sgr.lora_pool_stats(dw.pool)["free_pages"] == 100 + 2 * r5
    with pytest.raises(sgr.LoraError) as ei:
        sgr.lora_pool_evict(dw.pool, 5)
    assert ei.value.status == -5
    rank, scale, A, B = wl.adapters[5][0]
    sgr.lora_pool_load(dw.pool, 5, 0, rank, A, B, scale)
    with pytest.raises(sgr.LoraError) as ei:
        sgr.lora_pool_load(dw.pool, 5, 0, rank, A, B, scale)     # already loaded
    assert ei.value.status == -5
    big = np.zeros((64, h), np.uint16)
    free_before = sgr.lora_pool_stats(dw.pool)["free_pages"]
    sgr.lora_pool_evict(dw.pool, 7)
    free_mid = sgr.lora_pool_stats(dw.pool)["free_pages"]
    if free_mid < 128:
        with pytest.raises(sgr.LoraError) as ei:
            sgr.lora_pool_load(dw.pool, 7, 0, 64, big, big, 1.0)
        assert ei.value.status == -4
        assert sgr.lora_pool_stats(dw.pool)["free_pages"] == free_mid     # failed load: no side effect
    with pytest.raises(sgr.LoraError) as ei:
        sgr.lora_pool_load(dw.pool, 7, 0, 65, big, big, 1.0)
    assert ei.value.status == -3
    assert free_before <= free_mid
    dw.close()


def test_shrink_rejects_t_rows_that_are_not_16_byte_aligned():
    """The K-split sum stores four rank columns at once: t must be 16-byte aligned
    with ld_t and module_stride_t multiples of 4 (checked before any launch)."""
    wl = W.c2_bgmv_decode(draw_w=False, h=256, n_tokens=40)
    dw = DeviceWorkload(wl, device=0)
    dw.build_segments()
    x = dw._xp(dw.x_off[0])
    t = torch.zeros(wl.n_tokens * 20 + 8, dtype=torch.float32, device=dw.dev)
    bad = [(t.data_ptr() + 4, 16, 0), (t, 17, 0), (t, 18, 0)]
    for tp, ld, ms in bad:
        with pytest.raises(sgr.LoraError) as ei:
            sgr.lora_shrink(dw.pool, 0, 1, x, 256, 0, dw.seg, tp, ld, ms, dw.ws, dw.ws_bytes)
        assert ei.value.status == -1
    sgr.lora_shrink(dw.pool, 0, 1, x, 256, 0, dw.seg, t, 20, 0, dw.ws, dw.ws_bytes)   # aligned: accepted
    torch.cuda.synchronize()
    dw.close()


# ----------------------------------------------------------------- exact cases
@pytest.mark.parametrize("mode", ["sgmv", "bgmv"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rank1_fingerprint_bit_exact(mode, dtype):
    """A_a = e_j, B_a = e_k, scale 1, y0 = 0: y_i = x_i[j_a] in column k_a, exactly."""
    wl = W.fingerprint_rank1(dtype=dtype, n_tokens=300, h=256)
    wl.ids[100:190] = 4      # one long segment, so the matrix-core path runs too
    say(f"fingerprint {mode} {dtype}")
    dw, ys = run(wl, mode)
    exp = lo.lora_delta(wl, 0)
    assert np.array_equal(ys[0], exp)
    dw.close()


@pytest.mark.parametrize("mode", ["sgmv", "bgmv"])
def test_integer_inputs_bit_exact_f32(mode):
    wl = W.integer_exact(n_tokens=200, h=128, n_slots=6, max_rank=4)
    wl.ids[30:130] = 2
    say(f"integer exact {mode}")
    dw, ys = run(wl, mode)
    assert np.array_equal(ys[0], lo.apply_to_y0(wl, 0))
    dw.close()


def test_integer_inputs_bit_exact_bf16_matrix_cores():
    """bf16 inputs with |y| <= 256 stay exact; long segments take the matrix-core path."""
    wl = W.integer_exact(n_tokens=256, h=128, n_slots=3, dtype="bf16", ranks=[1, 2, 1], scale=1.0)
    rng = np.random.default_rng(0)
    for s in range(3):
        r, sc, A, B = wl.adapters[s][0]
        A = W.to_bf16_bits(rng.integers(-1, 2, (r, 128)).astype(np.float32))
        B = W.to_bf16_bits(rng.integers(-1, 2, (r, 128)).astype(np.float32))
        wl.adapters[s][0] = (r, sc, A, B)
    wl.x[0] = W.to_bf16_bits(rng.integers(-1, 2, (256, 128)).astype(np.float32))
    wl.y0[0] = W.to_bf16_bits(rng.integers(-4, 5, (256, 128)).astype(np.float32))
    wl.ids[:] = np.repeat([0, 1, 2, -1], 64)
    exp = lo.apply_to_y0(wl, 0)
    assert np.max(np.abs(exp)) <= 256
    for mode in ("sgmv", "bgmv"):
        dw, ys = run(wl, mode)
        assert np.array_equal(ys[0], exp), mode
        dw.close()


# ----------------------------------------------------------------- configs at tolerance
@pytest.mark.parametrize("mode", ["sgmv", "bgmv"])
def test_c1_tiny_f32(mode):
    wl = W.c1_tiny_f32()
    say(f"C1 {mode}")
    dw, ys = run(wl, mode)
    ref = lo.apply_to_y0(wl, 0)
    assert_close(ys[0], ref, "f32", "C1")
    neg = wl.ids < 0
    assert np.array_equal(ys[0][neg], lo.decode(wl.y0[0], "f32")[neg])     # id -1: y untouched
    dw.close()


@pytest.mark.parametrize("mode", ["bgmv", "sgmv"])
def test_c2_bgmv_decode(mode):
    wl = W.c2_bgmv_decode()
    say(f"C2 {mode}")
    dw, ys = run(wl, mode)
    assert_close(ys[0], lo.apply_to_y0(wl, 0), "bf16", "C2")
    dw.close()


def test_c2_delta_tight_fp32_output():
    """y0 = 0 in fp32: the kernel's adapter term against the oracle's, at fp32 accuracy."""
    wl = W.c2_bgmv_decode()
    for mode in ("bgmv", "sgmv"):
        dw = DeviceWorkload(wl, y_dtype="f32")
        dw.zero_y()
        dw.bgmv_step() if mode == "bgmv" else dw.sgmv_step()
        torch.cuda.synchronize()
        got = from_device(dw.y_of(0)).astype(np.float64)
        ref = lo.lora_delta(wl, 0)
        assert rel_l2(got, ref) <= 1e-5, mode
        dw.close()


def test_c3_reduced_mixed_paths():
    """512 tokens in 8 segments of 32..128: short ones on GEMV, long ones on matrix cores."""
    wl = W.c3_sgmv_prefill(h=512, units=(2, 8), total_units=32)
    say(f"C3 reduced, lengths {wl.notes['segment_lengths'].tolist()}")
    for mode in ("sgmv", "bgmv"):
        dw, ys = run(wl, mode)
        for m in range(4):
            assert_close(ys[m], lo.apply_to_y0(wl, m), "bf16", f"C3r {mode} m{m}")
        dw.close()


@pytest.mark.parametrize("rank", [32, 64])
def test_shared_x_high_rank_sub_ranges(rank):
    """q, k, v share x on pools of rank 32 and 64 at h = 4096: the matrix-core shrink runs two or
    four 16-column tiles per module for three modules at once, K split across workgroups, and
    each split's A rows staged in LDS as two or four sub-ranges; short segments share the launch."""
    wl = W.c3_sgmv_prefill(h=4096, rank=rank, units=(2, 8), total_units=32)
    say(f"shared x, rank {rank}, lengths {wl.notes['segment_lengths'].tolist()}")
    dw, ys = run(wl, "sgmv")
    for m in range(4):
        assert_close(ys[m], lo.apply_to_y0(wl, m), "bf16", f"rank {rank} m{m}")
    dw.close()


def test_c3_delta_tight_fp32_output_matrix_cores():
    """y0 = 0 in fp32 on a batch whose long segments run on the matrix cores: the
    bf16 MFMA expand multiplies by t itself (t as three exact bf16 parts), so the
    adapter term matches the oracle at fp32 accuracy."""
    wl = W.c3_sgmv_prefill(h=512, units=(2, 8), total_units=32)
    assert max(wl.notes["segment_lengths"]) >= 64
    for mode in ("sgmv", "bgmv"):
        dw = DeviceWorkload(wl, y_dtype="f32")
        dw.zero_y()
        dw.sgmv_step() if mode == "sgmv" else dw.bgmv_step()
        torch.cuda.synchronize()
        for m in range(4):
            got = from_device(dw.y_of(m)).astype(np.float64)
            assert rel_l2(got, lo.lora_delta(wl, m)) <= 1e-5, (mode, m)
        dw.close()


def test_mixed_rank_fp32_output_large_lds():
    """The mixed-rank batch (ranks up to 64) with y0 = 0 in fp32: the matrix-core expand then
    needs 78 KiB of LDS (above the 64 KiB default, so the library raises the kernel's limit),
    and the adapter term of every token, prefill or decode, matches the oracle at fp32 accuracy."""
    wl = W.c4_mixed_rank(h=1024, draw_w=False)
    dw = DeviceWorkload(wl, y_dtype="f32")
    dw.zero_y()
    dw.sgmv_step()
    torch.cuda.synchronize()
    got = from_device(dw.y_of(0)).astype(np.float64)
    assert rel_l2(got, lo.lora_delta(wl, 0)) <= 1e-5
    dw.close()


def test_wide_rows_in_several_pages():
    """h = 8192 (the GEMV shrink stages x in two slices) with pages of 2048
    elements (four pages per adapter row), on both GEMV paths."""
    import dataclasses
    wl = dataclasses.replace(W.c2_bgmv_decode(h=8192, n_tokens=24, n_slots=8), page_elems=2048)
    say("wide rows, 4 pages per row")
    for mode in ("bgmv", "sgmv"):
        dw, ys = run(wl, mode)
        assert_close(ys[0], lo.apply_to_y0(wl, 0), "bf16", f"wide {mode}")
        dw.close()


def test_c3_t_tight():
    wl = W.c3_sgmv_prefill(h=512, units=(2, 8), total_units=32)
    dw = DeviceWorkload(wl)
    dw.build_segments()
    dw.shrink()
    torch.cuda.synchronize()
    for m in range(4):
        t = dw.t_of(m).cpu().numpy().astype(np.float64)[:, :16]
        ref = lo.shrink_t(wl, m)[:, :16]
        assert rel_l2(t, ref) <= 1e-5, m
    dw.close()


def test_c4_mixed_rank():
    wl = W.c4_mixed_rank()
    say("C4")
    for mode in ("sgmv", "bgmv"):
        dw, ys = run(wl, mode)
        assert_close(ys[0], lo.apply_to_y0(wl, 0), "bf16", f"C4 {mode}")
        dw.close()


def _sample_tokens(wl, k, seed):
    rng = np.random.default_rng(seed)
    toks = set(rng.choice(wl.n_tokens, k, replace=False).tolist())
    toks.update(range(0, 70))                      # a whole tile and its ragged neighbour
    return np.array(sorted(toks))


def test_c3_full_size_sampled():
    wl = W.c3_sgmv_prefill(draw_w=False)
    say("C3 full")
    dw, ys = run(wl, "sgmv")
    toks = _sample_tokens(wl, 300, 1)
    for m in range(4):
        assert_close(ys[m][toks], lo.apply_to_y0(wl, m, toks), "bf16", f"C3 m{m}")
    dw.close()


def test_c5_full_size_sampled():
    wl = W.c5_encoder_step(draw_w=False)
    say("C5 full")
    dw, ys = run(wl, "sgmv")
    toks = _sample_tokens(wl, 400, 2)
    for m in range(4):
        assert_close(ys[m][toks], lo.apply_to_y0(wl, m, toks), "bf16", f"C5 m{m}")
    dw.close()


# ----------------------------------------------------------------- invariances
def test_run_twice_bitwise_identical():
    wl = W.c3_sgmv_prefill(h=512, units=(2, 8), total_units=32)
    outs = []
    for _ in range(2):
        dw, ys = run(wl, "sgmv")
        outs.append(ys)
        dw.close()
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_page_placement_invariance():
    """The same adapters in a fragmented pool (other pages) give bit-identical y."""
    wl = W.c4_mixed_rank(h=256, prefill_len=64, draw_w=False)
    dw1, y1 = run(wl, "sgmv")
    dw1.close()
    dw2 = DeviceWorkload(wl, extra_pages=600, load=True)
    # fragment: evict every other slot, fill holes with junk, reload the evicted adapters
    rng = np.random.default_rng(1)
    for s in range(0, wl.n_slots, 2):
        sgr.lora_pool_evict(dw2.pool, s)
    junk = []
    for s in range(0, wl.n_slots, 2):
        r = 8
        A = W.to_bf16_bits(rng.normal(0, 1, (r, 256)).astype(np.float32))
        sgr.lora_pool_load(dw2.pool, s, 0, r, A, A, 1.0)
        junk.append(s)
    for s in junk:
        sgr.lora_pool_evict(dw2.pool, s)
    for s in range(0, wl.n_slots, 2):
        r, sc, A, B = wl.adapters[s][0]
        sgr.lora_pool_load(dw2.pool, s, 0, r, A, B, sc)
    _, _, p_new = sgr.lora_pool_read(dw2.pool, 0, 0, max_pages=8)
    dw2.sgmv_step()
    torch.cuda.synchronize()
    y2 = lo.decode(from_device(dw2.y_of(0)), "bf16")
    assert np.array_equal(y1[0], y2)
    dw2.close()
    assert len(p_new) == 8


def test_zero_padding_invariance():
    """Rank r vs the same adapter padded with zero rows to r' gives bit-identical y."""
    wl = W.c4_mixed_rank(h=256, prefill_len=64, draw_w=False)
    dw1, y1 = run(wl, "sgmv")
    dw1.close()
    import copy
    wl2 = copy.copy(wl)
    pad = []
    for row in wl.adapters:
        r, s, A, B = row[0]
        r2 = min(64, r + 8)
        A2 = np.zeros((r2, A.shape[1]), A.dtype); A2[:r] = A
        B2 = np.zeros((r2, B.shape[1]), B.dtype); B2[:r] = B
        pad.append([(r2, s, A2, B2)])
    wl2.adapters = pad
    for mode in ("sgmv", "bgmv"):
        dwa, ya = run(wl, mode)
        dwb, yb = run(wl2, mode)
        assert np.array_equal(ya[0], yb[0]), mode
        dwa.close()
        dwb.close()


def test_bad_ids_leave_rows_untouched():
    wl = W.c2_bgmv_decode(h=256, n_tokens=40)
    wl.ids = wl.ids.copy()
    wl.ids[[3, 9, 17]] = [-5, 32, 1000]
    for mode in ("sgmv", "bgmv"):
        dw, ys = run(wl, mode)
        st, meta = sgr.lora_segments_check(dw.seg)
        assert st == -8 and meta[sgr.META["n_bad"]] == 3
        y0 = lo.decode(wl.y0[0], "bf16")
        assert np.array_equal(ys[0][[3, 9, 17]], y0[[3, 9, 17]])
        assert_close(ys[0], lo.apply_to_y0(wl, 0), "bf16", mode)
        dw.close()


@pytest.mark.parametrize("mode", ["bgmv", "sgmv"])
@pytest.mark.parametrize("n_modules", [12, 24, 33, 40])
def test_module_groups_with_short_tail(n_modules, mode):
    """A GEMV launch over 8 or more modules runs its modules in groups of up to
    32: one group of 12 or 24, or a full group and a short last one (1 or 8
    modules), must each match the oracle."""
    wl = W.c2_bgmv_decode(n_modules=n_modules, h=512, n_tokens=40)
    dw, ys = run(wl, mode)
    for m in range(n_modules):
        assert_close(ys[m], lo.apply_to_y0(wl, m), "bf16", f"{mode} m{m}")
    dw.close()


def test_c2_decode_128_modules_full_size_sampled():
    """The default decode batch: 64 tokens over 128 modules of 4096 x 4096 in one
    launch straight from the ids (the launch the decode bench times), in one bgmv
    after the segment build, and through shrink and expand (four groups of 32
    modules); modules at every group edge against the oracle."""
    wl = W.c2_bgmv_decode(n_modules=128, draw_w=False)
    for mode in ("bgmv_ids", "bgmv", "sgmv"):
        say(f"C2 x128 full {mode}")
        dw, ys = run(wl, mode)
        for m in (0, 1, 31, 32, 63, 64, 95, 96, 126, 127):
            assert_close(ys[m], lo.apply_to_y0(wl, m), "bf16", f"C2x128 {mode} m{m}")
        dw.close()


def test_multi_module_one_launch():
    """Eight decode modules with their own x and y in one bgmv launch and one sgmv pass."""
    wl = W.c2_bgmv_decode(n_modules=8, h=512, n_tokens=48)
    for mode in ("bgmv", "sgmv"):
        dw, ys = run(wl, mode)
        for m in range(8):
            assert_close(ys[m], lo.apply_to_y0(wl, m), "bf16", f"{mode} m{m}")
        dw.close()
