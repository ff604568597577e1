"""The seeded generators: determinism and the structure each workload promises (CPU)."""
import numpy as np
import pytest

import workloads as W


def _same(a, b):
    assert a.name == b.name and np.array_equal(a.ids, b.ids)
    for p, q in zip(a.x, b.x):
        assert np.array_equal(p, q)
    for p, q in zip(a.y0, b.y0):
        assert np.array_equal(p, q)
    for ra, rb in zip(a.adapters, b.adapters):
        for p, q in zip(ra, rb):
            assert p[0] == q[0] and p[1] == q[1]
            assert np.array_equal(p[2], q[2]) and np.array_equal(p[3], q[3])


@pytest.mark.parametrize("gen", [W.c1_tiny_f32,
                                 lambda: W.c2_bgmv_decode(h=256),
                                 lambda: W.c4_mixed_rank(h=128, prefill_len=32)])
def test_deterministic(gen):
    _same(gen(), gen())


def test_bf16_rounding_is_nearest_even():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.0e-3], np.float32)
    bits = W.to_bf16_bits(v)
    # 1+2^-8 is a tie between 1 and 1+2^-7: even mantissa (1.0) wins;
    # 1+3*2^-8 is a tie between 1+2^-7 and 1+2^-6: even is 1+2^-6
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == 1.0 + 2 ** -6 and back[3] == -2.5
    assert abs(back[4] - 3.0e-3) <= 3.0e-3 * 2 ** -8


def test_c1_structure():
    wl = W.c1_tiny_f32()
    assert wl.n_tokens == 16 and wl.dtype == "f32" and wl.page_elems == 64
    b = wl.notes["segment_bounds"]
    assert b[0] == 0 and b[-1] == 16 and np.all(np.diff(b) > 0) and len(b) == 5
    segs = wl.notes["segment_ids"]
    assert segs.count(-1) == 1 and len({s for s in segs if s >= 0}) == 3
    assert all(a[0] == 4 and a[1] == 2.0 for row in wl.adapters for a in row)


def test_c3_segment_lengths():
    wl = W.c3_sgmv_prefill(h=64, draw_w=False)
    L = wl.notes["segment_lengths"]
    assert L.sum() == 4096 and np.all(L % 16 == 0) and L.min() >= 128 and L.max() <= 1024
    assert sorted(wl.notes["segment_slots"].tolist()) == list(range(8))
    assert [m.x_group for m in wl.modules] == [0, 0, 0, 1]


def test_c4_structure():
    wl = W.c4_mixed_rank(h=128, draw_w=False)
    assert wl.n_tokens == 4 * 256 + 48
    for k in range(4):
        assert len(set(wl.ids[k * 256:(k + 1) * 256].tolist())) == 1
    ranks = {a[0] for row in wl.adapters for a in row}
    assert ranks <= {8, 16, 32, 64} and len(ranks) >= 3
    for row in wl.adapters:
        assert row[0][1] == 32.0 / row[0][0]


def test_zipf_slot0_hottest():
    rng = np.random.default_rng(0)
    ids = W.zipf_ids(rng, 20000, 32, 1.1)
    counts = np.bincount(ids, minlength=32)
    assert counts[0] == counts.max() and ids.min() >= 0 and ids.max() < 32
    cdf = W.finite_zipf_cdf(32, 1.1)
    assert abs(counts[0] / 20000 - cdf[0]) < 0.02
