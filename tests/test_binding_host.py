"""The Python binding refuses tensors of the wrong shape, dtype or layout
before anything reaches the C ABI (no GPU needed: the checks run on host
tensors, before any device pointer is taken).

The C ABI receives bare pointers and cannot see buffer sizes, so a wrongly
sized or typed tensor would otherwise be read or written out of bounds by the
kernels.
"""
import pytest
import torch

from mamba_ssd_scan_chunk_amd import binding as bd

B, L, H, P, G, N = 2, 40, 4, 16, 2, 32


def _prefill_args(dtype=torch.bfloat16):
    f32 = torch.float32
    return dict(x=torch.zeros(B, L, H, P, dtype=dtype), dt=torch.zeros(B, L, H, dtype=f32),
                A_log=torch.zeros(H, dtype=f32), Bm=torch.zeros(B, L, G, N, dtype=dtype),
                Cm=torch.zeros(B, L, G, N, dtype=dtype), D=torch.zeros(H, dtype=f32))


def _call_prefill(**over):
    a = _prefill_args()
    kw = {k: over.pop(k) for k in list(over) if k not in a}
    a.update(over)
    return bd.ssd_prefill(a["x"], a["dt"], a["A_log"], a["Bm"], a["Cm"], a["D"], Q=32, **kw)


def test_valid_host_tensors_reach_the_device_check():
    with pytest.raises(ValueError, match="must live on the GPU"):
        _call_prefill()


@pytest.mark.parametrize("over,msg", [
    (dict(dt=torch.zeros(B, L, H, dtype=torch.bfloat16)), "dt must be torch.float32"),
    (dict(dt=torch.zeros(B, L + 1, H)), r"dt must have shape"),
    (dict(A_log=torch.zeros(H + 1)), r"A_log must have shape"),
    (dict(A_log=torch.zeros(H, dtype=torch.float64)), "A_log must be torch.float32"),
    (dict(D=torch.zeros(H, dtype=torch.bfloat16)), "D must be torch.float32"),
    (dict(Bm=torch.zeros(B, L - 1, G, N, dtype=torch.bfloat16)), r"Bm must have shape"),
    (dict(Cm=torch.zeros(B, L, G, N, dtype=torch.float32)), "Cm must be torch.bfloat16"),
    (dict(Cm=torch.zeros(B, L, G, N + 1, dtype=torch.bfloat16)), r"Cm must have shape"),
    (dict(init_state=torch.zeros(B, H, P, N, dtype=torch.bfloat16)), "init_state must be torch.float32"),
    (dict(init_state=torch.zeros(B, H, N, P)), r"init_state must have shape"),
    (dict(y=torch.zeros(B, L, H, P, dtype=torch.float32)), "y must be torch.bfloat16"),
    (dict(y=torch.zeros(B, L, H, P + 1, dtype=torch.bfloat16)[..., :P]), "y must be contiguous"),
    (dict(final_state=torch.zeros(B, H, P, N - 1)), r"final_state must have shape"),
    (dict(workspace=torch.zeros(8, dtype=torch.uint8)), r"workspace holds 8 bytes"),
    (dict(workspace=torch.zeros(1 << 20, dtype=torch.float32)), "workspace must be a contiguous 1-D uint8"),
    (dict(x=torch.zeros(B, L, H * P, dtype=torch.bfloat16)), r"x must be \[B,L,H,P\]"),
    (dict(x=torch.zeros(B, L, H, P, dtype=torch.float16)), "unsupported activation dtype"),
])
def test_prefill_refuses(over, msg):
    with pytest.raises((ValueError, TypeError), match=msg):
        _call_prefill(**over)


def test_prefill_refuses_a_strided_x():
    x = torch.zeros(B, L, H, 2 * P, dtype=torch.bfloat16)[..., :P]
    with pytest.raises(ValueError, match="x must be contiguous"):
        _call_prefill(x=x)


def _varlen_args():
    T, f32, bf = 100, torch.float32, torch.bfloat16
    return dict(x=torch.zeros(T, H, P, dtype=bf), dt=torch.zeros(T, H), A_log=torch.zeros(H),
                Bm=torch.zeros(T, G, N, dtype=bf), Cm=torch.zeros(T, G, N, dtype=bf), D=torch.zeros(H, dtype=f32),
                cu_seqlens=torch.tensor([0, 30, 100], dtype=torch.int32))


@pytest.mark.parametrize("over,msg", [
    (dict(), "must live on the GPU"),
    (dict(dt=torch.zeros(99, H)), r"dt must have shape"),
    (dict(Cm=torch.zeros(100, G, N)), "Cm must be torch.bfloat16"),
    (dict(cu_seqlens=torch.tensor([0, 100], dtype=torch.int64)), "cu_seqlens must be int32"),
    (dict(init_state=torch.zeros(3, H, P, N)), r"init_state must have shape"),
    (dict(final_state=torch.zeros(2, H, P, N, dtype=torch.float64)), "final_state must be torch.float32"),
])
def test_varlen_refuses(over, msg):
    a = _varlen_args()
    kw = {k: over.pop(k) for k in list(over) if k in ("init_state", "final_state")}
    a.update(over)
    with pytest.raises((ValueError, TypeError), match=msg):
        bd.ssd_prefill_varlen(a["x"], a["dt"], a["A_log"], a["Bm"], a["Cm"], a["D"], a["cu_seqlens"], Q=256, **kw)


def _decode(stride=0, **over):
    bf, f32 = torch.bfloat16, torch.float32
    C = H * P + 2 * G * N
    row = torch.zeros(B, C, dtype=bf)
    if stride:
        a = dict(x_t=row[:, :H * P], B_t=row[:, H * P:H * P + G * N], C_t=row[:, H * P + G * N:])
    else:
        a = dict(x_t=torch.zeros(B, H * P, dtype=bf), B_t=torch.zeros(B, G * N, dtype=bf),
                 C_t=torch.zeros(B, G * N, dtype=bf))
    a.update(dt_t=torch.zeros(B, H), A_log=torch.zeros(H), D=torch.zeros(H, dtype=f32),
             ssm_state=torch.zeros(B, H, P, N))
    kw = dict(in_stride=stride, G=G)
    for k in list(over):
        (a if k in a else kw)[k] = over.pop(k)
    return bd.ssd_decode_step(a["x_t"], a["dt_t"], a["A_log"], a["B_t"], a["C_t"], a["D"], a["ssm_state"], **kw)


@pytest.mark.parametrize("stride", [0, H * P + 2 * G * N])
def test_decode_valid_host_tensors_reach_the_device_check(stride):
    with pytest.raises(ValueError, match="must live on the GPU"):
        _decode(stride)


@pytest.mark.parametrize("over,msg", [
    (dict(ssm_state=torch.zeros(B, H, P, N, dtype=torch.bfloat16)), "ssm_state must be torch.float32"),
    (dict(ssm_state=torch.zeros(B, H, N, P).transpose(2, 3)), "ssm_state must be contiguous"),
    (dict(dt_t=torch.zeros(B, H, dtype=torch.bfloat16)), "dt_t must be torch.float32"),
    (dict(dt_t=torch.zeros(B, H + 1)), r"dt_t must have shape"),
    (dict(D=torch.zeros(H - 1)), r"D must have shape"),
    (dict(x_t=torch.zeros(B, H * P - 1, dtype=torch.bfloat16)), "x_t must be dense"),
    (dict(x_t=torch.zeros(B, 2 * H * P, dtype=torch.bfloat16)[:, ::2]), "x_t must be dense"),
    (dict(B_t=torch.zeros(B, G * N, dtype=torch.float32)), "B_t must be torch.bfloat16"),
    (dict(C_t=torch.zeros(B, G * N + 8, dtype=torch.bfloat16)), "C_t must be dense"),
    (dict(y_t=torch.zeros(B, H, P)), "y_t must be torch.bfloat16"),
    (dict(y_t=torch.zeros(B, H, P - 1, dtype=torch.bfloat16)), r"y_t must have shape"),
    (dict(H=H + 1), "H, P, N given as"),
    (dict(conv_state_in=torch.zeros(B, H * P + 2 * G * N, 3, dtype=torch.bfloat16)), "conv_state_out and conv_w"),
])
def test_decode_refuses(over, msg):
    with pytest.raises((ValueError, TypeError), match=msg):
        _decode(0, **over)


def test_decode_refuses_a_view_with_another_row_stride():
    C = H * P + 2 * G * N
    wide = torch.zeros(B, C + 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="x_t must have row stride"):
        _decode(C, x_t=wide[:, :H * P])


def test_decode_refuses_bad_conv_tensors():
    C, K = H * P + 2 * G * N, 4
    ok = dict(conv_state_in=torch.zeros(B, C, K - 1, dtype=torch.bfloat16),
              conv_state_out=torch.zeros(B, C, K - 1, dtype=torch.bfloat16),
              conv_w=torch.zeros(C, K, dtype=torch.bfloat16), K=K, activation=1)
    with pytest.raises(ValueError, match="must live on the GPU"):
        _decode(0, **dict(ok))
    for key, bad, msg in [("conv_state_out", torch.zeros(B, C, K - 1), "conv_state_out must be torch.bfloat16"),
                          ("conv_w", torch.zeros(C, K + 1, dtype=torch.bfloat16), r"conv_w must have shape"),
                          ("conv_state_in", torch.zeros(B, C - 1, K - 1, dtype=torch.bfloat16), "conv_state_in must")]:
        kw = dict(ok)
        kw[key] = bad
        with pytest.raises(ValueError, match=msg):
            _decode(0, **kw)


@pytest.mark.parametrize("over,msg", [
    (dict(), "must live on the GPU"),
    (dict(xBC=torch.zeros(B, 5, 33, dtype=torch.bfloat16)), r"xBC must have shape"),
    (dict(conv_w=torch.zeros(32, 3, dtype=torch.bfloat16)), r"conv_w must have shape"),
    (dict(conv_b=torch.zeros(32)), "conv_b must be torch.bfloat16"),
    (dict(out=torch.zeros(B, 4, 32, dtype=torch.bfloat16)), r"out must have shape"),
])
def test_conv_refuses(over, msg):
    a = dict(conv_state=torch.zeros(B, 32, 3, dtype=torch.bfloat16), xBC=torch.zeros(B, 5, 32, dtype=torch.bfloat16),
             conv_w=torch.zeros(32, 4, dtype=torch.bfloat16))
    kw = {k: over.pop(k) for k in list(over) if k not in a}
    a.update(over)
    with pytest.raises(ValueError, match=msg):
        bd.conv_state_update(a["conv_state"], a["xBC"], a["conv_w"], **kw)


@pytest.mark.parametrize("over,msg", [
    (dict(), "must live on the GPU"),
    (dict(xBC=torch.zeros(50, 40, dtype=torch.bfloat16)), r"xBC must have shape"),
    (dict(cu_seqlens=torch.tensor([0, 50], dtype=torch.int32)), r"cu_seqlens must have shape"),
    (dict(workspace=torch.zeros(4, dtype=torch.uint8)), "workspace holds 4 bytes"),
])
def test_conv_varlen_refuses(over, msg):
    a = dict(conv_state=torch.zeros(2, 32, 3, dtype=torch.bfloat16), xBC=torch.zeros(50, 32, dtype=torch.bfloat16),
             cu_seqlens=torch.tensor([0, 20, 50], dtype=torch.int32), conv_w=torch.zeros(32, 4, dtype=torch.bfloat16))
    kw = {k: over.pop(k) for k in list(over) if k not in a}
    a.update(over)
    with pytest.raises(ValueError, match=msg):
        bd.conv_state_update_varlen(a["conv_state"], a["xBC"], a["cu_seqlens"], a["conv_w"], **kw)


def test_norm_refuses_a_wrong_output():
    y = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"out must have shape"):
        bd.ssd_gated_rmsnorm(y, group=64, out=torch.zeros(4, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must be torch.bfloat16"):
        bd.ssd_gated_rmsnorm(y, group=64, out=torch.zeros(4, 64))
