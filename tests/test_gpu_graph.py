"""Graph capture: the segment build and the apply calls enqueue only kernels on the
caller's stream (no memsets, no host synchronization), so a serving loop can capture
them in a HIP graph.  Each replay, with eager work between replays, must give the
eager result bit for bit (every reduction has a fixed order)."""
import pytest

import workloads as W

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _replays_match_eager(wl, step):
    from segmented_gathered_rank_amd.harness import DeviceWorkload
    dw = DeviceWorkload(wl, device=0)
    dw.reset_y()
    step(dw)
    torch.cuda.synchronize()
    ref = [dw.y_of(m).clone() for m in range(wl.n_modules)]
    g = torch.cuda.CUDAGraph()
    capture = torch.cuda.Stream()
    dw.reset_y()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=capture):
        step(dw)
    for rep in range(3):
        dw.reset_y()                                 # eager work between the replays
        x_before = dw.x.clone()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for m in range(wl.n_modules):
            assert torch.equal(dw.y_of(m), ref[m]), (rep, m)
        assert torch.equal(dw.x, x_before)
    dw.close()


def test_graph_replay_bgmv():
    """Segment build + fused BGMV over four modules, captured and replayed."""
    _replays_match_eager(W.c2_bgmv_decode(n_modules=4, h=512, n_tokens=48, draw_w=False),
                         lambda dw: dw.bgmv_step())


def test_graph_replay_shrink_expand():
    """Segment build + shrink (one launch of tiles and units, then the split reduce) + expand,
    on a batch with short and long segments, captured and replayed."""
    _replays_match_eager(W.c3_sgmv_prefill(h=512, units=(2, 8), total_units=32, draw_w=False),
                         lambda dw: dw.sgmv_step())


def test_graph_replay_bgmv_ids():
    """The fused BGMV straight from the ids (one launch, its segment build in LDS) over four
    modules, units split into column ranges, captured and replayed; and a one-module call."""
    _replays_match_eager(W.c2_bgmv_decode(n_modules=4, h=4096, n_tokens=48, draw_w=False),
                         lambda dw: dw.bgmv_ids())
    _replays_match_eager(W.c2_bgmv_decode(n_modules=1, h=4096, n_tokens=64, draw_w=False),
                         lambda dw: dw.bgmv_ids())
