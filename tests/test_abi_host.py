"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

Every call here fails argument validation, which runs on the host before any
HIP call, so nothing reaches the device.
"""
import ctypes
import os
import re
import subprocess

import pytest

from mamba_ssd_scan_chunk_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bd.LIB_PATH):
        from mamba_ssd_scan_chunk_amd import build

        build.build(verbose=False)
    return bd.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"}


def test_header_declares_the_abi():
    assert _declared_functions() == set(bd.SIGNATURES)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.check_output(["nm", "-D", "--defined-only", bd.LIB_PATH], text=True)
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert _declared_functions() <= exported
    for name in _declared_functions():
        assert hasattr(lib, name)


def test_debug_knobs_validate_their_arguments(lib):
    assert lib.ssd_debug_handoff_jitter(-1) == bd.SSD_ERR_INVALID_ARG
    assert lib.ssd_debug_handoff_jitter(100001) == bd.SSD_ERR_INVALID_ARG
    assert lib.ssd_debug_handoff_jitter(0) == 0
    assert lib.ssd_debug_handoff_ticks(-1) == 0
    for bad in (-2, 2):
        assert lib.ssd_debug_packed_form(bad) == bd.SSD_ERR_INVALID_ARG
    for ok in (0, 1, -1):
        assert lib.ssd_debug_packed_form(ok) == 0


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert bd.ssd_status_string(code)
    assert bd.ssd_status_string(-99) == "unknown status"
    assert bd.ssd_last_hip_error() == 0


# fake, well-aligned, non-overlapping device addresses (never dereferenced)
_BASE = 0x7F0000000000
_STEP = 1 << 34


def _addr(i, off=0):
    return _BASE + i * _STEP + off


def _prefill(lib, B=1, L=64, H=2, P=16, G=1, N=16, Q=32, dtype=0, **over):
    ptrs = dict(x=_addr(0), dt=_addr(1), A_log=_addr(2), Bm=_addr(3), Cm=_addr(4), D=_addr(5),
                init=_addr(6), y=_addr(7), final=_addr(8), ws=_addr(9))
    ws_bytes = over.pop("ws_bytes", 1 << 40)
    ptrs.update(over)
    return lib.ssd_prefill(B, L, H, P, G, N, Q, dtype, ptrs["x"], ptrs["dt"], ptrs["A_log"], ptrs["Bm"],
                           ptrs["Cm"], ptrs["D"], ptrs["init"], ptrs["y"], ptrs["final"], ptrs["ws"],
                           ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(G=3, H=4), bd.SSD_ERR_INVALID_ARG),          # G does not divide H
    (dict(B=0), bd.SSD_ERR_INVALID_ARG),
    (dict(L=-1), bd.SSD_ERR_INVALID_ARG),
    (dict(P=0), bd.SSD_ERR_INVALID_ARG),
    (dict(Q=0), bd.SSD_ERR_INVALID_ARG),
    (dict(dtype=7), bd.SSD_ERR_INVALID_ARG),
    (dict(x=None), bd.SSD_ERR_INVALID_ARG),
    (dict(dt=None), bd.SSD_ERR_INVALID_ARG),
    (dict(A_log=None), bd.SSD_ERR_INVALID_ARG),
    (dict(y=None), bd.SSD_ERR_INVALID_ARG),
    (dict(P=257), bd.SSD_ERR_UNSUPPORTED),
    (dict(N=512), bd.SSD_ERR_UNSUPPORTED),
    (dict(Q=1025), bd.SSD_ERR_UNSUPPORTED),
    (dict(x=_addr(0, 2)), bd.SSD_ERR_ALIGNMENT),
    (dict(y=_addr(7, 8)), bd.SSD_ERR_ALIGNMENT),
    (dict(final=_addr(8, 4)), bd.SSD_ERR_ALIGNMENT),
    (dict(ws=_addr(9, 16)), bd.SSD_ERR_ALIGNMENT),
    (dict(y=_addr(0, 64)), bd.SSD_ERR_INVALID_ARG),      # y overlaps x
    (dict(final=_addr(4, 0)), bd.SSD_ERR_INVALID_ARG),   # final_state overlaps Cm
    (dict(final=_addr(6, 16)), bd.SSD_ERR_INVALID_ARG),  # partial overlap with init_state
    (dict(ws=_addr(3, 0)), bd.SSD_ERR_INVALID_ARG),      # workspace overlaps Bm
    (dict(ws=None), bd.SSD_ERR_WORKSPACE),
    (dict(ws_bytes=16), bd.SSD_ERR_WORKSPACE),
])
def test_prefill_rejects(lib, kw, code):
    assert _prefill(lib, **kw) == code


def _prefill_raw(lib, B=1, L=64, H=2, P=16, G=1, N=16, Q=32, dtype=0, dt_min=0.001, dt_max=0.1, **over):
    ptrs = dict(x=_addr(0), dt=_addr(1), bias=_addr(10), A_log=_addr(2), Bm=_addr(3), Cm=_addr(4), D=_addr(5),
                init=_addr(6), y=_addr(7), final=_addr(8), ws=_addr(9))
    ptrs.update(over)
    return lib.ssd_prefill_dt_raw(B, L, H, P, G, N, Q, dtype, ptrs["x"], ptrs["dt"], ptrs["bias"], dt_min, dt_max,
                                  ptrs["A_log"], ptrs["Bm"], ptrs["Cm"], ptrs["D"], ptrs["init"], ptrs["y"],
                                  ptrs["final"], ptrs["ws"], 1 << 40, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt_min=-0.1), bd.SSD_ERR_INVALID_ARG),
    (dict(dt_min=0.2, dt_max=0.1), bd.SSD_ERR_INVALID_ARG),
    (dict(dt_min=float("nan")), bd.SSD_ERR_INVALID_ARG),
    (dict(dt_max=float("nan")), bd.SSD_ERR_INVALID_ARG),
    (dict(bias=_addr(10, 2)), bd.SSD_ERR_ALIGNMENT),
    (dict(y=_addr(10, 0)), bd.SSD_ERR_INVALID_ARG),     # y overlaps dt_bias
    (dict(G=3, H=4), bd.SSD_ERR_INVALID_ARG),          # the checks of ssd_prefill apply
    (dict(dt=None), bd.SSD_ERR_INVALID_ARG),
])
def test_prefill_dt_raw_rejects(lib, kw, code):
    assert _prefill_raw(lib, **kw) == code


def test_prefill_dt_raw_accepts_open_limits(lib):
    # no bias, dt_max = +inf: valid; L = 0 without outputs returns before any HIP call
    assert _prefill_raw(lib, L=0, bias=None, dt_min=0.0, dt_max=float("inf"), final=None, x=None, y=None) == bd.SSD_OK


def test_prefill_empty_sequence_without_outputs_is_a_no_op(lib):
    # L = 0 and no final_state: nothing to do, returns before any HIP call
    assert _prefill(lib, L=0, final=None, x=None, y=None) == bd.SSD_OK


def test_workspace_query(lib):
    assert lib.ssd_prefill_workspace_bytes(1, 0, 2, 16, 1, 16, 64, 0) == 0
    n1 = lib.ssd_prefill_workspace_bytes(1, 256, 2, 16, 1, 16, 64, 0)
    n2 = lib.ssd_prefill_workspace_bytes(1, 257, 2, 16, 1, 16, 64, 0)  # one more (ragged) chunk
    assert 0 < n1 < n2 and n1 % 256 == 0
    assert n1 >= 4 * 2 * 16 * 16 * 4  # at least one fp32 state per head-chunk
    assert lib.ssd_prefill_workspace_bytes(1, 256, 3, 16, 2, 16, 64, 0) == ctypes.c_size_t(-1).value


def _decode(lib, B=2, H=2, P=16, G=1, N=16, dtype=0, K=4, act=1, stride=0, **over):
    p = dict(x=_addr(0), dt=_addr(1), A_log=_addr(2), Bt=_addr(3), Ct=_addr(4), D=_addr(5), state=_addr(6),
             y=_addr(7), cin=_addr(8), cout=_addr(9), w=_addr(10), b=_addr(11))
    p.update(over)
    return lib.ssd_decode_step(B, H, P, G, N, dtype, p["x"], p["dt"], p["A_log"], p["Bt"], p["Ct"], p["D"],
                               p["state"], p["y"], stride, p["cin"], p["cout"], p["w"], p["b"], K, act, None)


@pytest.mark.parametrize("kw,code", [
    (dict(G=3, H=4), bd.SSD_ERR_INVALID_ARG),
    (dict(B=0), bd.SSD_ERR_INVALID_ARG),
    (dict(state=None), bd.SSD_ERR_INVALID_ARG),
    (dict(y=None), bd.SSD_ERR_INVALID_ARG),
    (dict(K=1), bd.SSD_ERR_INVALID_ARG),
    (dict(K=9), bd.SSD_ERR_INVALID_ARG),
    (dict(act=2), bd.SSD_ERR_INVALID_ARG),
    (dict(cout=None), bd.SSD_ERR_INVALID_ARG),
    (dict(w=None), bd.SSD_ERR_INVALID_ARG),
    (dict(stride=-1), bd.SSD_ERR_INVALID_ARG),
    (dict(stride=8), bd.SSD_ERR_INVALID_ARG),          # shorter than H*P
    (dict(cout=_addr(8)), bd.SSD_ERR_INVALID_ARG),     # conv out aliases conv in
    (dict(y=_addr(6, 64)), bd.SSD_ERR_INVALID_ARG),    # y inside the state
    (dict(state=_addr(0, 0)), bd.SSD_ERR_INVALID_ARG),  # state overlaps x_t
    (dict(N=48), bd.SSD_ERR_UNSUPPORTED),
    (dict(N=512), bd.SSD_ERR_UNSUPPORTED),
    (dict(P=2048), bd.SSD_ERR_UNSUPPORTED),
    (dict(state=_addr(6, 4)), bd.SSD_ERR_ALIGNMENT),
    (dict(x=_addr(0, 2)), bd.SSD_ERR_ALIGNMENT),        # fp32 element misaligned
])
def test_decode_rejects(lib, kw, code):
    assert _decode(lib, **kw) == code


def _varlen(lib, B=3, T=500, H=2, P=64, G=1, N=128, Q=256, dtype=1, ws_bytes=1 << 40, **over):
    p = dict(cu=_addr(13), x=_addr(0), dt=_addr(1), A_log=_addr(2), Bm=_addr(3), Cm=_addr(4), D=_addr(5),
             init=_addr(6), y=_addr(7), final=_addr(8), ws=_addr(9))
    p.update(over)
    return lib.ssd_prefill_varlen(B, T, H, P, G, N, Q, dtype, p["cu"], p["x"], p["dt"], p["A_log"], p["Bm"],
                                  p["Cm"], p["D"], p["init"], p["y"], p["final"], p["ws"], ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), bd.SSD_ERR_INVALID_ARG),
    (dict(cu=_addr(13, 2)), bd.SSD_ERR_ALIGNMENT),
    (dict(y=_addr(13, 0)), bd.SSD_ERR_INVALID_ARG),      # y overlaps cu_seqlens
    (dict(final=_addr(13, 0)), bd.SSD_ERR_INVALID_ARG),  # final_state overlaps cu_seqlens
    (dict(ws=_addr(13, 0)), bd.SSD_ERR_INVALID_ARG),     # workspace overlaps cu_seqlens
    (dict(T=-1), bd.SSD_ERR_INVALID_ARG),
    (dict(B=0), bd.SSD_ERR_INVALID_ARG),
    (dict(G=3, H=4), bd.SSD_ERR_INVALID_ARG),
    (dict(ws_bytes=1024), bd.SSD_ERR_WORKSPACE),
    (dict(ws=None), bd.SSD_ERR_WORKSPACE),
    (dict(Q=2048), bd.SSD_ERR_UNSUPPORTED),
])
def test_varlen_rejects(lib, kw, code):
    assert _varlen(lib, **kw) == code


def test_mfma_longer_chunks_use_the_256_token_workspace(lib):
    w256 = lib.ssd_prefill_workspace_bytes(1, 4096, 80, 64, 1, 128, 256, 1)
    assert lib.ssd_prefill_workspace_bytes(1, 4096, 80, 64, 1, 128, 512, 1) == w256
    assert lib.ssd_prefill_workspace_bytes(1, 4096, 80, 64, 1, 128, 1024, 1) == w256
    # not a multiple of 256, or not the MFMA shape: the vector path's workspace
    assert lib.ssd_prefill_workspace_bytes(1, 4096, 80, 64, 1, 128, 384, 1) != w256
    assert lib.ssd_prefill_workspace_bytes(1, 4096, 80, 64, 1, 64, 512, 1) != \
        lib.ssd_prefill_workspace_bytes(1, 4096, 80, 64, 1, 64, 256, 1)


@pytest.mark.parametrize("kw,code", [
    (dict(dt_min=-1.0), bd.SSD_ERR_INVALID_ARG),
    (dict(dt_max=float("nan")), bd.SSD_ERR_INVALID_ARG),
    (dict(bias=_addr(12, 2)), bd.SSD_ERR_ALIGNMENT),
    (dict(cu=None), bd.SSD_ERR_INVALID_ARG),
    (dict(y=_addr(12, 0)), bd.SSD_ERR_INVALID_ARG),  # y overlaps dt_bias
])
def test_varlen_dt_raw_rejects(lib, kw, code):
    p = dict(cu=_addr(13), x=_addr(0), dt=_addr(1), bias=_addr(12), A_log=_addr(2), Bm=_addr(3), Cm=_addr(4),
             D=_addr(5), init=_addr(6), y=_addr(7), final=_addr(8), ws=_addr(9))
    kw = dict(kw)
    lo, hi = kw.pop("dt_min", 0.0), kw.pop("dt_max", 1.0)
    p.update(kw)
    rc = lib.ssd_prefill_varlen_dt_raw(3, 500, 2, 64, 1, 128, 256, 1, p["cu"], p["x"], p["dt"], p["bias"], lo, hi,
                                       p["A_log"], p["Bm"], p["Cm"], p["D"], p["init"], p["y"], p["final"], p["ws"],
                                       1 << 40, None)
    assert rc == code


def test_varlen_workspace_bytes(lib):
    n = lib.ssd_prefill_varlen_workspace_bytes(3, 500, 2, 64, 1, 128, 256, 1)
    # chunk slots: 500 / 256 + 3 = 4; the slot and sequence tables come last
    per_slot = lib.ssd_prefill_workspace_bytes(1, 256, 2, 64, 1, 128, 256, 1)
    assert abs(n - (4 * per_slot + 4 * 16 + 3 * 8)) <= 8 * 256  # up to 256-byte padding per region
    assert lib.ssd_prefill_varlen_workspace_bytes(3, 0, 2, 64, 1, 128, 256, 1) == 0
    assert lib.ssd_prefill_varlen_workspace_bytes(0, 10, 2, 64, 1, 128, 256, 1) == ctypes.c_size_t(-1).value


def _decode_raw(lib, B=2, H=2, P=16, G=1, N=16, dtype=0, K=4, act=1, dt_min=0.0, dt_max=1.0, **over):
    p = dict(x=_addr(0), dt=_addr(1), bias=_addr(12), A_log=_addr(2), Bt=_addr(3), Ct=_addr(4), D=_addr(5),
             state=_addr(6), y=_addr(7), cin=_addr(8), cout=_addr(9), w=_addr(10), b=_addr(11))
    p.update(over)
    return lib.ssd_decode_step_dt_raw(B, H, P, G, N, dtype, p["x"], p["dt"], p["bias"], dt_min, dt_max, p["A_log"],
                                      p["Bt"], p["Ct"], p["D"], p["state"], p["y"], 0, p["cin"], p["cout"], p["w"],
                                      p["b"], K, act, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt_max=-1.0), bd.SSD_ERR_INVALID_ARG),
    (dict(dt_min=float("nan")), bd.SSD_ERR_INVALID_ARG),
    (dict(bias=_addr(12, 1)), bd.SSD_ERR_ALIGNMENT),
    (dict(state=_addr(12, 0)), bd.SSD_ERR_INVALID_ARG),  # state overlaps dt_bias
    (dict(K=1), bd.SSD_ERR_INVALID_ARG),                 # the checks of ssd_decode_step apply
])
def test_decode_dt_raw_rejects(lib, kw, code):
    assert _decode_raw(lib, **kw) == code


def _conv(lib, B=2, T=8, C=40, K=4, dtype=1, act=1, **over):
    p = dict(state=_addr(0), x=_addr(1), w=_addr(2), b=_addr(3), out=_addr(4))
    p.update(over)
    return lib.conv_state_update(B, T, C, K, dtype, p["state"], p["x"], p["w"], p["b"], act, p["out"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(K=1), bd.SSD_ERR_INVALID_ARG),
    (dict(K=9), bd.SSD_ERR_INVALID_ARG),
    (dict(T=-1), bd.SSD_ERR_INVALID_ARG),
    (dict(C=0), bd.SSD_ERR_INVALID_ARG),
    (dict(dtype=3), bd.SSD_ERR_INVALID_ARG),
    (dict(act=5), bd.SSD_ERR_INVALID_ARG),
    (dict(state=None), bd.SSD_ERR_INVALID_ARG),
    (dict(w=None), bd.SSD_ERR_INVALID_ARG),
    (dict(x=None), bd.SSD_ERR_INVALID_ARG),
    (dict(out=_addr(1, 32)), bd.SSD_ERR_INVALID_ARG),   # out overlaps xBC
    (dict(state=_addr(1, 0)), bd.SSD_ERR_INVALID_ARG),  # cache overlaps xBC
    (dict(T=65536 * 16), bd.SSD_ERR_UNSUPPORTED),
    (dict(state=_addr(0, 1)), bd.SSD_ERR_ALIGNMENT),
])
def test_conv_rejects(lib, kw, code):
    assert _conv(lib, **kw) == code


def _conv_vl(lib, B=2, T=40, C=64, K=4, dtype=1, act=1, ws_bytes=1 << 30, **over):
    p = dict(cu=_addr(5), state=_addr(0), x=_addr(1), w=_addr(2), b=_addr(3), out=_addr(4), ws=_addr(6))
    p.update(over)
    return lib.conv_state_update_varlen(B, T, C, K, dtype, p["cu"], p["state"], p["x"], p["w"], p["b"], act,
                                        p["out"], p["ws"], ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(cu=None), bd.SSD_ERR_INVALID_ARG),
    (dict(B=0), bd.SSD_ERR_INVALID_ARG),
    (dict(K=9), bd.SSD_ERR_INVALID_ARG),
    (dict(state=None), bd.SSD_ERR_INVALID_ARG),
    (dict(out=_addr(5, 0)), bd.SSD_ERR_INVALID_ARG),    # out overlaps cu_seqlens
    (dict(ws=_addr(1, 256)), bd.SSD_ERR_INVALID_ARG),   # workspace overlaps xBC
    (dict(C=60), bd.SSD_ERR_UNSUPPORTED),               # not a multiple of 8 bf16
    (dict(x=_addr(1, 8)), bd.SSD_ERR_ALIGNMENT),
    (dict(cu=_addr(5, 2)), bd.SSD_ERR_ALIGNMENT),
    (dict(ws=_addr(6, 64)), bd.SSD_ERR_ALIGNMENT),
    (dict(ws_bytes=16), bd.SSD_ERR_WORKSPACE),
    (dict(ws=None), bd.SSD_ERR_WORKSPACE),
])
def test_conv_varlen_rejects(lib, kw, code):
    assert _conv_vl(lib, **kw) == code


def test_conv_varlen_workspace(lib):
    assert _conv_vl(lib, T=0, x=None, ws=None) == bd.SSD_OK
    assert lib.conv_state_update_varlen_workspace_bytes(2, 0) == 0
    assert lib.conv_state_update_varlen_workspace_bytes(2, 40) >= (40 // 8 + 2) * 16 + 2 * 16
    assert lib.conv_state_update_varlen_workspace_bytes(0, 40) == ctypes.c_size_t(-1).value


def test_conv_zero_tokens_is_a_no_op(lib):
    assert _conv(lib, T=0, x=None) == bd.SSD_OK


def _norm(lib, rows=4, D=5120, group=5120, dtype=1, eps=1e-5, z_stride=None, **over):
    p = dict(y=_addr(0), z=_addr(1), w=_addr(2), out=_addr(3))
    p.update(over)
    zs = D if z_stride is None else z_stride
    return lib.ssd_gated_rmsnorm(rows, D, group, dtype, p["y"], p["z"], zs, p["w"], eps, p["out"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), bd.SSD_ERR_INVALID_ARG),
    (dict(D=0), bd.SSD_ERR_INVALID_ARG),
    (dict(group=0), bd.SSD_ERR_INVALID_ARG),
    (dict(group=1000), bd.SSD_ERR_INVALID_ARG),            # does not divide D
    (dict(dtype=2), bd.SSD_ERR_INVALID_ARG),
    (dict(eps=-1e-6), bd.SSD_ERR_INVALID_ARG),
    (dict(eps=float("nan")), bd.SSD_ERR_INVALID_ARG),
    (dict(eps=float("inf")), bd.SSD_ERR_INVALID_ARG),
    (dict(y=None), bd.SSD_ERR_INVALID_ARG),
    (dict(out=None), bd.SSD_ERR_INVALID_ARG),
    (dict(z_stride=5000), bd.SSD_ERR_INVALID_ARG),         # rows of z shorter than D
    (dict(out=_addr(0, 1024)), bd.SSD_ERR_INVALID_ARG),    # out partly overlaps y
    (dict(out=_addr(1, 0)), bd.SSD_ERR_INVALID_ARG),       # out overlaps z
    (dict(out=_addr(2, 16)), bd.SSD_ERR_INVALID_ARG),      # out overlaps norm_w
    (dict(D=20, group=20), bd.SSD_ERR_UNSUPPORTED),         # group not a multiple of 8 bf16
    (dict(D=960, group=96), bd.SSD_ERR_UNSUPPORTED),       # 12 vectors: neither 2^k <= 64 nor 64m
    (dict(D=5120, group=640), bd.SSD_ERR_UNSUPPORTED),     # 80 vectors
    (dict(D=16384 + 512, group=512), bd.SSD_ERR_UNSUPPORTED),  # row longer than 2048 vectors
    (dict(dtype=0, D=8192 + 256, group=256), bd.SSD_ERR_UNSUPPORTED),
    (dict(y=_addr(0, 8)), bd.SSD_ERR_ALIGNMENT),
    (dict(z=_addr(1, 8)), bd.SSD_ERR_ALIGNMENT),
    (dict(w=_addr(2, 4)), bd.SSD_ERR_ALIGNMENT),
    (dict(z_stride=5124), bd.SSD_ERR_ALIGNMENT),            # row stride not a multiple of 8 bf16
])
def test_gated_rmsnorm_rejects(lib, kw, code):
    assert _norm(lib, **kw) == code


def test_gated_rmsnorm_accepts_in_place_and_empty(lib):
    # rows = 0 returns before any HIP call; out == y (in place) is allowed
    assert _norm(lib, rows=0, out=_addr(0)) == bd.SSD_OK
    assert _norm(lib, rows=0, y=None, out=None, z=None, w=None) == bd.SSD_OK


def test_binding_refuses_host_tensors(lib):
    import torch

    x = torch.zeros(1, 4, 1, 16)
    with pytest.raises(ValueError):
        bd.ssd_prefill(x, torch.zeros(1, 4, 1), torch.zeros(1), torch.zeros(1, 4, 1, 16),
                       torch.zeros(1, 4, 1, 16), Q=16)


def test_product_path_does_not_touch_the_oracle():
    """The package and its sources never import or link the oracle."""
    pkg = os.path.join(ROOT, "mamba_ssd_scan_chunk_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "from oracle" not in text, f
                assert "ssd_oracle" not in text, f


def test_stage_timing_queries_without_a_timed_call(lib):
    """Before any timed ssd_prefill call there is nothing to report, and the
    query rejects a missing count pointer; neither touches the device."""
    n = ctypes.c_int(-1)
    assert lib.ssd_stage_times(None, 0, ctypes.byref(n)) == bd.SSD_OK
    assert n.value == 0
    assert lib.ssd_stage_times(None, 0, None) == bd.SSD_ERR_INVALID_ARG
    assert lib.ssd_stage_times(None, 4, ctypes.byref(n)) == bd.SSD_ERR_INVALID_ARG
    assert lib.ssd_stage_name(0) is None and lib.ssd_stage_name(-1) is None


def test_packed_chained_workspace_stops_at_the_item_record_limit(lib):
    # Packed sequences of the chained shape (B*H >= 192) hold both prefill
    # forms' buffers and the item order.  An item record holds a slot below
    # 2^22; from that many slots on the call runs the four-kernel form alone,
    # so its workspace drops by the chained form's regions, then grows again.
    H, P, G, N, Q = 192, 64, 1, 128, 256
    cap_T = ((1 << 22) - 1) * Q  # slots = T / Q + B = 2^22 at B = 1
    below, at, above = (lib.ssd_prefill_varlen_workspace_bytes(1, T, H, P, G, N, Q, bd.SSD_BF16)
                        for T in (cap_T - Q, cap_T, cap_T + Q))
    assert at < below and at < above
    # below the bound of 192 chains the four-kernel layout alone
    assert lib.ssd_prefill_varlen_workspace_bytes(1, 4096, 191, P, G, N, Q, bd.SSD_BF16) < \
        lib.ssd_prefill_varlen_workspace_bytes(1, 4096, 192, P, G, N, Q, bd.SSD_BF16)
