"""ssd_prefill_noalloc: the prefill without a workspace argument, for callers
that cannot allocate device memory.  Its scratch is the library's fixed
per-GPU buffer, which keeps the last call's contents; it must give exactly
the bits of ssd_prefill (same kernels) on consecutive calls whose second is
smaller than the first, and the oracle's result within the dtype's
tolerance.  The host-side checks need no GPU."""
import ctypes

import pytest
import torch

from mamba_ssd_scan_chunk_amd import binding as bd
from mamba_ssd_scan_chunk_amd import synth
from tests.gpu_utils import TOL_BF16, TOL_F32, announce, dev, rel_err

_BASE, _STEP = 0x7F0000000000, 1 << 36


def _noalloc_raw(B, L, H, P, G, N, Q, dtype, **over):
    ptrs = dict(x=_BASE, dt=_BASE + _STEP, A_log=_BASE + 2 * _STEP, Bm=_BASE + 3 * _STEP, Cm=_BASE + 4 * _STEP,
                D=_BASE + 5 * _STEP, init=None, y=_BASE + 7 * _STEP, final=_BASE + 8 * _STEP)
    ptrs.update(over)
    return bd.lib().ssd_prefill_noalloc(B, L, H, P, G, N, Q, dtype, ptrs["x"], ptrs["dt"], ptrs["A_log"],
                                        ptrs["Bm"], ptrs["Cm"], ptrs["D"], ptrs["init"], ptrs["y"], ptrs["final"],
                                        None)


def test_noalloc_scratch_size_matches_the_header():
    import os
    import re
    hdr = open(os.path.join(os.path.dirname(bd.__file__), "..", "include", "ssd.h")).read()
    m = re.search(r"#define SSD_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == bd.NOALLOC_SCRATCH_BYTES


def test_noalloc_rejects_before_any_hip_call():
    """Too large for the fixed scratch (the B = 8, L = 16384 layer needs about
    2 GB), and the argument checks of ssd_prefill: all on the host."""
    assert bd.ssd_prefill_workspace_bytes(8, 16384, 80, 64, 1, 128, 256, bd.SSD_BF16) > bd.NOALLOC_SCRATCH_BYTES
    assert _noalloc_raw(8, 16384, 80, 64, 1, 128, 256, bd.SSD_BF16) == bd.SSD_ERR_TOO_LARGE
    assert _noalloc_raw(1, 64, 4, 16, 3, 16, 32, 0) == bd.SSD_ERR_INVALID_ARG      # G does not divide H
    assert _noalloc_raw(1, 64, 2, 16, 1, 16, 32, 0, x=None) == bd.SSD_ERR_INVALID_ARG
    assert _noalloc_raw(1, 64, 2, 16, 1, 16, 32, 0, y=_BASE + 2) == bd.SSD_ERR_ALIGNMENT
    assert _noalloc_raw(1, 64, 2, 16, 1, 16, 32, 0, y=_BASE + 64) == bd.SSD_ERR_INVALID_ARG  # y overlaps x
    assert "no-allocation" in bd.ssd_status_string(bd.SSD_ERR_TOO_LARGE)
    # the 2.7B-shaped layer at B = 1, L = 4096 fits
    assert bd.ssd_prefill_workspace_bytes(1, 4096, 80, 64, 1, 128, 256, bd.SSD_BF16) <= bd.NOALLOC_SCRATCH_BYTES


# (name, B, L, H, P, G, N, Q, dtype): each pair is run in this order, the
# second call smaller than the first
PAIRS = [
    [("mamba2-2.7b-prefill", 1, 4096, 80, 64, 1, 128, 256, "bf16"), ("mfma-small", 2, 700, 3, 64, 1, 128, 256, "bf16")],
    [("vector-f32", 2, 900, 4, 16, 2, 32, 64, "f32"), ("vector-f32-small", 1, 130, 2, 16, 1, 32, 64, "f32")],
    # the chained single pass (B*H >= 192): control block and hand-off slots in the scratch
    [("chain-b4h80", 4, 2048, 80, 64, 1, 128, 256, "bf16"), ("chain-b16h16", 16, 300, 16, 64, 1, 128, 256, "bf16")],
]


@pytest.mark.gpu
@pytest.mark.parametrize("pair", PAIRS, ids=["mfma", "vector", "chain"])
def test_noalloc_equals_prefill_on_consecutive_calls(oracle, pair):
    for i, (name, B, L, H, P, G, N, Q, dtype) in enumerate(pair):
        d = synth.make_prefill(B, L, H, P, G, N, dtype, seed=900 + i)
        init = synth.make_state(B, H, P, N, seed=901 + i, scale=0.5)
        dd, initd = dev(d), init.cuda()
        announce("noalloc", name)
        y_ref, fs_ref = bd.ssd_prefill(dd["x"], dd["dt"], dd["A_log"], dd["Bm"], dd["Cm"], dd["D"], initd, Q=Q)
        y = torch.full_like(y_ref, 7.0)
        fs = torch.full_like(fs_ref, 7.0)
        bd.ssd_prefill_noalloc(dd["x"], dd["dt"], dd["A_log"], dd["Bm"], dd["Cm"], dd["D"], initd, Q=Q, y=y,
                               final_state=fs)
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), name
        assert torch.equal(fs, fs_ref), name
        y_o, fs_o = oracle.ssd_scan(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], init)
        tol = TOL_F32 if dtype == "f32" else TOL_BF16
        assert rel_err(y, y_o) <= tol, name
        assert rel_err(fs, fs_o) <= tol, name
