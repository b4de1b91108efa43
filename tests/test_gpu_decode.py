"""GPU parity of ssd_decode_step (fused conv + state update + readout) and
conv_state_update against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from mamba_ssd_scan_chunk_amd import binding as bd
from mamba_ssd_scan_chunk_amd import synth
from tests.gpu_utils import TOL_BF16, TOL_F32, TOL_STATE, announce, f64, rel_err

pytestmark = pytest.mark.gpu


def _tol(dtype):
    return TOL_F32 if dtype == "f32" else TOL_BF16


def _setup(B, H, P, G, N, K, dtype, steps, seed, variant="spec", with_bias=False):
    C = H * P + 2 * G * N
    tdt = synth.torch_dtype(dtype)
    xbc, dts = synth.make_decode_stream(steps, B, H, P, G, N, dtype, seed, variant)
    w, bias = synth.make_conv(C, K, dtype, seed + 1, with_bias)
    pre = synth.make_prefill(B, 1, H, P, G, N, dtype, seed + 2, variant)
    state0 = synth.make_state(B, H, P, N, seed + 3, scale=0.3)
    conv0 = synth.make_tokens(B, K - 1, C, dtype, seed + 4).transpose(1, 2).contiguous()
    return dict(C=C, tdt=tdt, xbc=xbc, dts=dts, w=w, bias=bias, A_log=pre["A_log"], D=pre["D"],
                state0=state0, conv0=conv0)


def _run_steps(oracle, B, H, P, G, N, K, dtype, steps, seed, conv, raw_dt=None):
    """``raw_dt`` = (with_bias, dt_min, dt_max): the step is passed raw and
    preprocessed inside the kernel; the oracle gets dt_from_raw of it."""
    s = _setup(B, H, P, G, N, K, dtype, steps, seed=seed, with_bias=conv)
    kw, ref_dts = {}, s["dts"]
    if raw_dt is not None:
        with_bias, lo, hi = raw_dt
        raw, dt_bias = synth.make_dt_raw((steps, B), H, seed + 5)
        dt_bias = dt_bias if with_bias else None
        s["dts"] = raw
        ref_dts = oracle.dt_from_raw(raw, dt_bias, lo, hi)
        kw = dict(dt_raw=True, dt_bias=None if dt_bias is None else dt_bias.cuda(), dt_min=lo, dt_max=hi)
    C = s["C"]
    state = s["state0"].cuda()
    cin, cout = s["conv0"].cuda(), torch.empty_like(s["conv0"]).cuda()
    w = s["w"].cuda()
    bias = s["bias"].cuda() if s["bias"] is not None else None
    A_log, D = s["A_log"].cuda(), s["D"].cuda()
    ref_state, ref_conv = f64(s["state0"]), f64(s["conv0"])
    for t in range(steps):
        row = s["xbc"][t].cuda()  # [B, C] raw channels x | B | C
        dt = s["dts"][t].cuda()
        x_t, B_t, C_t = row[:, :H * P], row[:, H * P:H * P + G * N], row[:, H * P + G * N:]
        y = bd.ssd_decode_step(x_t, dt, A_log, B_t, C_t, D, state, in_stride=C, G=G,
                               conv_state_in=cin if conv else None, conv_state_out=cout if conv else None,
                               conv_w=w, conv_b=bias, K=K, activation=1, **kw)
        torch.cuda.synchronize()
        r = s["xbc"][t]
        y_ref, ref_state, new_conv = oracle.decode_step(
            r[:, :H * P], ref_dts[t], s["A_log"], r[:, H * P:H * P + G * N], r[:, H * P + G * N:],
            s["D"], ref_state, conv_state=ref_conv if conv else None, conv_w=s["w"], conv_b=s["bias"],
            activation=True)
        assert rel_err(y, y_ref) <= _tol(dtype), t
        assert rel_err(state, ref_state) <= TOL_STATE, t
        if conv:
            np.testing.assert_array_equal(f64(cout), new_conv)  # raw values, shifted exactly
            ref_conv = new_conv
            cin, cout = cout, cin


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("conv", [False, True])
def test_decode_steps_match_oracle(oracle, dtype, N, conv):
    """Small grid: blocks of 16-64 rows, ragged, heads of P=20 rows crossing
    block boundaries, two groups."""
    announce("decode", dtype, f"N={N}", f"conv={conv}")
    _run_steps(oracle, 2, 4, 20, 2, N, 4, dtype, 5, N + (100 if conv else 0), conv)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("conv", [False, True])
@pytest.mark.parametrize("raw_dt", [(True, 1e-3, 0.1), (False, 0.0, float("inf"))], ids=["bias-clip", "plain"])
def test_decode_dt_raw_matches_oracle(oracle, dtype, conv, raw_dt):
    """dt preprocessing fused into the decode step: softplus of the raw step
    plus a per-head bias, clipped (both bounds reached by the inputs), or
    softplus alone."""
    announce("decode dt_raw", dtype, f"conv={conv}", raw_dt)
    _run_steps(oracle, 2, 4, 20, 2, 128, 4, dtype, 4, 300 + conv, conv, raw_dt)
    _run_steps(oracle, 64, 16, 20, 2, 128, 4, dtype, 2, 310 + conv, conv, raw_dt)  # large-block launch


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_largest_head(oracle, dtype):
    """The largest shape the decode step takes: P = 1024, N = 256, K = 8."""
    announce("decode largest head", dtype)
    _run_steps(oracle, 2, 2, 1024, 1, 256, 8, dtype, 3, 77, True)


@pytest.mark.parametrize("K", [2, 3, 8])
def test_decode_conv_widths(oracle, K):
    """Conv widths other than 4 (the width taken from the arguments)."""
    announce("decode conv width", K)
    _run_steps(oracle, 2, 4, 20, 2, 128, K, "bf16", 3, 50 + K, True)


@pytest.mark.parametrize("dtype,N,K", [("bf16", 16, 4), ("bf16", 32, 4), ("bf16", 64, 4), ("bf16", 128, 4),
                                       ("f32", 128, 4), ("bf16", 128, 3), ("bf16", 256, 4)])
def test_decode_large_grid(oracle, dtype, N, K):
    """Enough blocks for the large-block launch (>= 1024 blocks of 4x the
    small-grid rows), with P=20 so that heads cross blocks and the last
    block of each group is ragged."""
    announce("decode large grid", dtype, f"N={N}", f"K={K}")
    _run_steps(oracle, 64, 16, 20, 2, N, K, dtype, 2, 200 + N + K, True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("conv", [False, True])
def test_decode_mid_grid(oracle, dtype, N, conv):
    """Between 64 and 128 workgroups of the largest blocks: the launch with
    blocks twice the smallest (B=5, H=16, P=20: heads cross blocks, the last
    block of each group is ragged, two groups)."""
    announce("decode mid grid", dtype, f"N={N}", f"conv={conv}")
    _run_steps(oracle, 5, 16, 20, 2, N, 4, dtype, 3, 400 + N + conv, conv)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_dense_separate_inputs(oracle, dtype):
    """in_stride = 0: x_t, B_t, C_t are separate dense tensors, no conv."""
    B, H, P, G, N = 3, 6, 64, 3, 128
    s = _setup(B, H, P, G, N, 4, dtype, 1, seed=7)
    r = s["xbc"][0]
    x_t, B_t, C_t = (r[:, :H * P].contiguous(), r[:, H * P:H * P + G * N].contiguous(),
                     r[:, H * P + G * N:].contiguous())
    state = s["state0"].cuda()
    announce("decode dense", dtype)
    y = bd.ssd_decode_step(x_t.cuda(), s["dts"][0].cuda(), s["A_log"].cuda(), B_t.cuda(), C_t.cuda(),
                           None, state)
    torch.cuda.synchronize()
    y_ref, st_ref, _ = oracle.decode_step(x_t, s["dts"][0], s["A_log"], B_t, C_t, None, s["state0"])
    assert rel_err(y, y_ref) <= _tol(dtype)
    assert rel_err(state, st_ref) <= TOL_STATE


# (batch, heads, sampled (b, h) pairs), one case per workgroup instance of
# the decode kernel: B*H*ceil(P/64) workgroups of 64 rows would be 24 for the
# 130M-shaped layer at B = 1 (16-row instance), 80 for the 2.7B-shaped layer
# at B = 1 (32-row instance), 160 at B = 2 and 1280 at B = 16 (64-row
# instance).  B = 16 is the batch the decode bench times; its pairs include
# heads in the first and the last workgroup of each batch element's group,
# the first and the last batch element, and workgroups on each of the eight
# XCDs (workgroup b*80 + h runs on XCD h mod 8).
DECODE_4096 = [
    (1, 24, [(0, 0), (0, 13), (0, 23)]),
    (1, 80, [(0, 0), (0, 37), (0, 79)]),
    (2, 80, [(0, 0), (0, 37), (1, 79), (1, 5)]),
    (16, 80, [(0, 0), (0, 79), (3, 41), (7, 78), (8, 2), (11, 61), (15, 79), (15, 0), (5, 11), (12, 68)]),
]


@pytest.mark.parametrize("variant", ["spec", "slow"])
@pytest.mark.parametrize("B,H,pairs", DECODE_4096, ids=["b1-h24", "b1", "b2", "b16"])
def test_decode_4096_steps_2p7b_shape(oracle, variant, B, H, pairs):
    """4096 consecutive fused decode steps of a 2.7B-shaped layer (H=80, P=64,
    N=128, conv C=5376, K=4, bf16 activations, fp32 state), and of the
    130M-shaped one (H=24).  The oracle starts from the same initial state
    bits and replays the same raw tokens for sampled (batch, head) pairs; the
    final fp32 state must agree to 1e-5."""
    P, G, N, K, steps = 64, 1, 128, 4, 4096
    w_ = synth.WORKLOADS["mamba2-2.7b-decode-b16" if H == 80 else "mamba2-130m-decode-b16"]
    assert (w_.H, w_.P, w_.N, w_.conv_channels) == (H, P, N, H * P + 2 * N)
    seed = 300 + (variant == "slow") + 2 * (B == 16) + 4 * (B == 1) + 8 * (H == 24)
    s = _setup(B, H, P, G, N, K, "bf16", steps, seed=seed, variant=variant)
    C = s["C"]
    announce("decode 4096", variant, f"B={B}")
    state = s["state0"].cuda()
    cin = torch.zeros_like(s["conv0"]).cuda()
    cout = torch.empty_like(cin)
    xbc, dts = s["xbc"].cuda(), s["dts"].cuda()
    w, A_log, D = s["w"].cuda(), s["A_log"].cuda(), s["D"].cuda()
    ys = torch.empty((steps, B, H, P), dtype=torch.bfloat16, device="cuda")
    for t in range(steps):
        row = xbc[t]
        bd.ssd_decode_step(row[:, :H * P], dts[t], A_log, row[:, H * P:H * P + N], row[:, H * P + N:], D,
                           state, y_t=ys[t], in_stride=C, G=G, conv_state_in=cin, conv_state_out=cout,
                           conv_w=w, K=K, activation=1)
        cin, cout = cout, cin
    torch.cuda.synchronize()
    # oracle: conv over the whole token stream (a FIR, so equal to stepping),
    # then the recurrence for sampled heads from the same initial state
    for b, h in pairs:
        stream = s["xbc"][:, b:b + 1, :].transpose(0, 1)  # [1, steps, C]
        _, out = oracle.conv_update(np.zeros((1, C, K - 1)), stream, s["w"], None, True)
        xs = out[:, :, h * P:(h + 1) * P].reshape(1, steps, 1, P)
        Bs = out[:, :, H * P:H * P + N].reshape(1, steps, 1, N)
        Cs = out[:, :, H * P + N:].reshape(1, steps, 1, N)
        y_ref, st_ref = oracle.ssd_scan(xs, s["dts"][:, b:b + 1, h:h + 1].transpose(0, 1), s["A_log"][h:h + 1],
                                        Bs, Cs, s["D"][h:h + 1], s["state0"][b:b + 1, h:h + 1])
        assert rel_err(state[b, h], st_ref[0, 0]) <= TOL_STATE, (b, h)
        assert rel_err(ys[:, b, h], y_ref[0, :, 0]) <= TOL_BF16, (b, h)
    np.testing.assert_array_equal(f64(cin), s["xbc"][-(K - 1):].permute(1, 2, 0).to(torch.float64).numpy())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("K", [2, 3, 4, 8])
@pytest.mark.parametrize("T", [1, 2, 5, 17, 100])
@pytest.mark.parametrize("C", [300, 304])
def test_conv_state_update_matches_oracle(oracle, dtype, K, T, C):
    """C = 304: 16-byte channel groups for both dtypes; C = 300: one channel
    per thread for bf16 (300 % 8 != 0), channel groups for fp32."""
    B = 2
    xbc = synth.make_tokens(B, T, C, dtype, seed=T * 10 + K)
    w, bias = synth.make_conv(C, K, dtype, seed=K, with_bias=(T % 2 == 1))
    st0 = synth.make_tokens(B, K - 1, C, dtype, seed=K + 50).transpose(1, 2).contiguous()
    st = st0.cuda()
    announce("conv", dtype, K, T)
    out = bd.conv_state_update(st, xbc.cuda(), w.cuda(), None if bias is None else bias.cuda(),
                               activation=int(T != 5))
    torch.cuda.synchronize()
    st_ref, out_ref = oracle.conv_update(st0, xbc, w, bias, T != 5)
    np.testing.assert_array_equal(f64(st), st_ref)
    assert rel_err(out, out_ref) <= (1e-6 if dtype == "f32" else 8e-3)


@pytest.mark.parametrize("K", [3, 4])
def test_conv_unaligned_tensors(oracle, K):
    """Tensors at 2-byte offsets take the one-channel-per-thread form; same
    result as the oracle."""
    B, C, T = 2, 304, 37
    xbc = synth.make_tokens(B, T, C, "bf16", seed=90 + K)
    w, bias = synth.make_conv(C, K, "bf16", seed=91 + K, with_bias=True)
    st0 = synth.make_tokens(B, K - 1, C, "bf16", seed=92 + K).transpose(1, 2).contiguous()
    announce("conv unaligned", K)
    # views one element into larger buffers: every pointer is 2 mod 16
    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
        v = buf[1:].view(t.shape)
        v.copy_(t.cuda())
        return v
    st, xd, wd, bd_ = shifted(st0), shifted(xbc), shifted(w), shifted(bias)
    outbuf = torch.empty(xbc.numel() + 1, dtype=xbc.dtype, device="cuda")
    out = outbuf[1:].view(xbc.shape)
    bd.conv_state_update(st, xd, wd, bd_, activation=1, out=out)
    torch.cuda.synchronize()
    st_ref, out_ref = oracle.conv_update(st0, xbc, w, bias, True)
    np.testing.assert_array_equal(f64(st), st_ref)
    assert rel_err(out, out_ref) <= 8e-3


def test_conv_prompt_then_steps_equals_one_pass(oracle):
    """Conv of a prompt from a zero cache, then token-by-token steps, equals
    one pass over the whole stream (and leaves the same cache)."""
    B, C, K, T1, T2 = 1, 5376, 4, 257, 9
    xbc = synth.make_tokens(B, T1 + T2, C, "bf16", seed=77)
    w, _ = synth.make_conv(C, K, "bf16", seed=78)
    xbc_d, w_d = xbc.cuda(), w.cuda()
    announce("conv prompt+steps")
    st_a = torch.zeros((B, C, K - 1), dtype=torch.bfloat16, device="cuda")
    out_a = bd.conv_state_update(st_a, xbc_d, w_d, activation=1)
    st_b = torch.zeros_like(st_a)
    outs = [bd.conv_state_update(st_b, xbc_d[:, :T1].contiguous(), w_d, activation=1)]
    for t in range(T1, T1 + T2):
        outs.append(bd.conv_state_update(st_b, xbc_d[:, t:t + 1].contiguous(), w_d, activation=1))
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, 1), out_a)
    assert torch.equal(st_a, st_b)
    _, out_ref = oracle.conv_update(np.zeros((B, C, K - 1)), xbc, w, None, True)
    assert rel_err(out_a, out_ref) <= 8e-3


def test_conv_cache_only(oracle):
    B, T, C, K = 1, 3, 64, 4  # T = K-1: whole cache replaced by the new tokens
    xbc = synth.make_tokens(B, T, C, "f32", seed=90)
    w, _ = synth.make_conv(C, K, "f32", seed=91)
    st = torch.ones((B, C, K - 1), device="cuda")
    announce("conv cache only")
    assert bd.conv_state_update(st, xbc.cuda(), w.cuda(), want_out=False) is None
    torch.cuda.synchronize()
    np.testing.assert_array_equal(f64(st), f64(xbc.transpose(1, 2)))


@pytest.mark.parametrize("B", [1, 16])
def test_cache_save_restore_continues_bit_for_bit(B):
    """The O(1) cache (ssm_state and conv_state) is the whole state of a
    generation: copied to the host after k decode steps, restored into fresh
    device buffers and continued for m more steps, it gives the outputs and
    the final cache of the uninterrupted k + m steps bit for bit (the
    functional cache and its update of bqwf.cn article §2.1-§2.2)."""
    H, P, G, N, K, k, m = 80, 64, 1, 128, 4, 7, 9
    s = _setup(B, H, P, G, N, K, "bf16", k + m, seed=340 + B)
    C = s["C"]
    xbc, dts = s["xbc"].cuda(), s["dts"].cuda()
    w, A_log, D = s["w"].cuda(), s["A_log"].cuda(), s["D"].cuda()

    def steps(state, cin, cout, t0, t1, ys):
        for t in range(t0, t1):
            row = xbc[t]
            bd.ssd_decode_step(row[:, :H * P], dts[t], A_log, row[:, H * P:H * P + N], row[:, H * P + N:], D,
                               state, y_t=ys[t], in_stride=C, G=G, conv_state_in=cin, conv_state_out=cout,
                               conv_w=w, K=K, activation=1)
            cin, cout = cout, cin
        return cin, cout

    announce("decode save/restore", f"B={B}")
    ys_a = torch.empty((k + m, B, H, P), dtype=torch.bfloat16, device="cuda")
    st_a = s["state0"].cuda()
    cin_a, _ = steps(st_a, s["conv0"].cuda(), torch.empty_like(s["conv0"]).cuda(), 0, k + m, ys_a)

    ys_b = torch.empty_like(ys_a)
    st_b = s["state0"].cuda()
    cin_b, _ = steps(st_b, s["conv0"].cuda(), torch.empty_like(s["conv0"]).cuda(), 0, k, ys_b)
    torch.cuda.synchronize()
    saved_state, saved_conv = st_b.cpu(), cin_b.cpu()  # the whole cache, on the host
    del st_b, cin_b
    torch.cuda.synchronize()
    st_c = torch.empty((B, H, P, N), dtype=torch.float32, device="cuda")
    st_c.copy_(saved_state)
    cin_c = torch.empty_like(s["conv0"]).cuda()
    cin_c.copy_(saved_conv)
    cin_c, _ = steps(st_c, cin_c, torch.empty_like(cin_c), k, k + m, ys_b)
    torch.cuda.synchronize()
    assert torch.equal(ys_b, ys_a)
    assert torch.equal(st_c, st_a)
    assert torch.equal(cin_c, cin_a)
