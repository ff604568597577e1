"""Host-side checks that need no GPU.

* the HIP library loads and exports every function include/lora.h declares;
* argument checks that run before any HIP call return their documented codes;
* the segment buffer layout and work-list bounds;
* the page allocator of the paged store, built with g++ under ASan/UBSan.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[a-z_0-9 \*]+?\b(lora_[a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    fns = declared_functions()
    for name in ["lora_build_segments", "lora_shrink", "lora_expand", "lora_apply_bgmv", "lora_pool_create",
                 "lora_pool_load", "lora_pool_evict", "lora_pool_destroy", "lora_pool_stats"]:
        assert name in fns


def test_library_exports_every_declared_symbol():
    import segmented_gathered_rank_amd as sgr
    out = subprocess.run(["nm", "-D", "--defined-only", sgr.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\sT\s(\S+)", out))
    missing = [f for f in declared_functions() if f not in exported]
    assert not missing, missing


def test_status_strings_and_version():
    import segmented_gathered_rank_amd as sgr
    assert sgr.lora_abi_version() == 8
    for code in sgr.STATUS:
        assert sgr.lora_status_str(code) and sgr.lora_status_str(code) != "unknown status"


def test_pool_create_rejects_bad_arguments_before_touching_a_device():
    import segmented_gathered_rank_amd as sgr
    bad = [
        (dict(page_elems=100), sgr.LoraError, -2),          # not a multiple of 64
        (dict(max_rank=65), sgr.LoraError, -3),             # above the rank cap
        (dict(max_rank=0), sgr.LoraError, -3),
        (dict(h_in=[4096 + 64]), sgr.LoraError, -2),        # not whole pages
        (dict(n_slots=0), sgr.LoraError, -1),
        (dict(n_slots=9000), sgr.LoraError, -1),
        (dict(wdtype=7), sgr.LoraError, -1),
    ]
    for kw, exc, code in bad:
        args = dict(device=0, wdtype=sgr.LORA_BF16, page_elems=4096, n_pages=8, n_slots=4, n_modules=1,
                    h_in=[4096], h_out=[4096], max_rank=16)
        args.update(kw)
        with pytest.raises(exc) as ei:
            sgr.lora_pool_create(**args)
        assert ei.value.status == code, kw


def test_apply_calls_reject_null_pool():
    import segmented_gathered_rank_amd as sgr
    seg = sgr.lora_segments()
    with pytest.raises(sgr.LoraError) as ei:
        sgr.lora_shrink(0, 0, 1, 16, 64, 0, seg, 16, 16, 0)
    assert ei.value.status == -1
    with pytest.raises(sgr.LoraError):
        sgr.lora_expand(0, 0, 1, 16, 16, 0, seg, 16, 64, 0, sgr.LORA_BF16)
    with pytest.raises(sgr.LoraError):
        sgr.lora_apply_bgmv(0, 0, 1, 16, 64, 0, seg, 16, 64, 0, sgr.LORA_BF16)
    with pytest.raises(sgr.LoraError):
        sgr.lora_build_segments(16, seg)           # n_slots 0 in an unbound struct


def test_segments_layout_and_bounds():
    import segmented_gathered_rank_amd as sgr
    for n, s in [(0, 4), (1, 1), (16, 4), (64, 32), (1072, 64), (4096, 8), (32768, 1024)]:
        nb = sgr.lora_segments_bytes(n, s)
        fake = 1 << 40                            # host-side layout only, never dereferenced
        seg = sgr.lora_segments()
        import ctypes
        st = sgr._lib.lora_segments_bind(fake, nb, n, s, ctypes.byref(seg))
        assert st == 0
        assert seg.max_segs == min(n, s)
        assert seg.max_units == (n + 3) // 4 + min(n, s)
        assert seg.max_tiles == (n + 63) // 64 + n // 64
        ptrs = [seg.perm, seg.seg_start, seg.seg_slot, seg.meta, seg.units, seg.tiles]
        assert all(p % 256 == 0 for p in ptrs) and ptrs == sorted(ptrs)
        assert seg.tiles + 8 * seg.max_tiles <= fake + nb
        if seg.n_chunks:   # the large-batch schedule's scratch follows the tiles
            assert seg.work % 256 == 0 and seg.work >= seg.tiles + 8 * seg.max_tiles
            assert seg.work + 4 * (2 * seg.n_chunks * s + s + seg.n_chunks) <= fake + nb
        else:
            assert seg.work is None
        assert sgr._lib.lora_segments_bind(fake, nb - 1, n, s, ctypes.byref(seg)) == -9
        assert sgr._lib.lora_segments_bind(fake + 16, nb, n, s, ctypes.byref(seg)) == -1


def _schedule(n, s):
    import ctypes
    import segmented_gathered_rank_amd as sgr
    seg = sgr.lora_segments()
    assert sgr._lib.lora_segments_bind(1 << 40, 1 << 40, n, s, ctypes.byref(seg)) == 0
    return seg.n_chunks


def test_segment_builder_schedule():
    """One workgroup up to 512 tokens per LDS histogram row (rows = min(16,
    16384 // n_slots - 1)), then chunks of >= 1024 tokens (a multiple of 64),
    at most 256 of them and at most 2**19 chunk-slot counters."""
    assert _schedule(8192, 64) == 0 and _schedule(8193, 64) == 9
    assert _schedule(512, 8192) == 0 and _schedule(513, 8192) == 1 and _schedule(600, 8192) == 1
    assert _schedule(7680, 1024) == 0 and _schedule(32768, 1024) == 32
    assert _schedule(20000, 8192) == 20            # 1024-token chunks, under the 2**19 / 8192 = 64 cap
    assert _schedule(1 << 20, 8192) == 64          # capped by the counters: chunks of 16384 tokens
    assert _schedule(1 << 24, 1) == 256            # capped at 256 chunks of 65536 tokens
    assert _schedule(131072, 300) == 128


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
@pytest.mark.parametrize("name", ["test_page_alloc", "test_launch_limits"])
def test_host_code_under_sanitizers(tmp_path, name):
    """The page allocator and the launch-size guard, built for the host with g++."""
    exe = tmp_path / name
    src = os.path.join(ROOT, "tests", "cpp", name + ".cpp")
    inc = os.path.join(ROOT, "segmented_gathered_rank_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", inc, src, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "ok" in r.stdout
