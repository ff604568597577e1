"""Helpers for the GPU tests: run the library on a workload, compare with the oracle."""
import sys

import numpy as np

from oracle import lora_oracle as lo


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run(wl, mode, y_dtype=None, **kw):
    """Runs one step from y = y0: 'sgmv' (the harness's choice of lora_apply_sgmv or
    lora_shrink + lora_expand), 'sgmv_calls' (always lora_shrink + lora_expand),
    'bgmv' (segment build + lora_apply_bgmv) or 'bgmv_ids' (lora_apply_bgmv_ids);
    returns (dw, y per module as float64)."""
    from segmented_gathered_rank_amd.harness import DeviceWorkload, from_device
    import torch
    dw = DeviceWorkload(wl, y_dtype=y_dtype, **kw)
    if mode == "sgmv":
        dw.sgmv_step()
    elif mode == "sgmv_calls":
        dw.build_segments()
        dw.shrink()
        dw.expand()
    elif mode == "bgmv_ids":
        dw.bgmv_ids()
    else:
        dw.bgmv_step()
    torch.cuda.synchronize()
    ys = [lo.decode(from_device(dw.y_of(m)), dw.y_dtype) for m in range(wl.n_modules)]
    return dw, ys


def rel_l2(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def assert_close(got, ref, dtype, what=""):
    """The parity bar: bf16 outputs rel-L2 <= 5e-3 and max-abs <= 2e-2 max|y|;
    fp32 outputs rel-L2 <= 1e-5.  Both computed over the whole tensor in fp64."""
    r = rel_l2(got, ref)
    if dtype == "bf16":
        m = float(np.max(np.abs(got - ref))) if got.size else 0.0
        lim = 2e-2 * float(np.max(np.abs(ref))) if ref.size else 0.0
        assert r <= 5e-3 and m <= lim, f"{what}: rel-L2 {r:.3e}, max-abs {m:.3e} (limit {lim:.3e})"
    else:
        assert r <= 1e-5, f"{what}: rel-L2 {r:.3e}"
    return r
