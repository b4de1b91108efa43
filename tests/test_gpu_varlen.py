"""GPU parity of ssd_prefill_varlen (sequences packed without padding)
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from mamba_ssd_scan_chunk_amd import binding as bd
from mamba_ssd_scan_chunk_amd import synth
from tests.gpu_utils import TOL_BF16, TOL_F32, announce, dev, rel_err

pytestmark = pytest.mark.gpu

PATHS = [
    # name, H, P, G, N, Q, dtype
    ("mfma", 4, 64, 2, 128, 256, "bf16"),
    ("vector-f32", 3, 16, 1, 16, 64, "f32"),
    ("mfma-q512", 2, 64, 1, 128, 512, "bf16"),
    ("vector-bf16-q512", 2, 64, 1, 64, 512, "bf16"),
]
MIXES = {
    # empty sequences, one token, chunk-size boundaries, ragged tails
    "edges": [0, 1, 255, 256, 257, 0, 700, 31],
    "one": [600],
    "many-short": [3, 17, 1, 64, 65, 9, 128, 40, 2, 90],
}


def _tol(dtype):
    return TOL_F32 if dtype == "f32" else TOL_BF16


def _run(d, Q, init=None):
    dd = dev(d)
    y, fs = bd.ssd_prefill_varlen(dd["x"], dd["dt"], dd["A_log"], dd["Bm"], dd["Cm"], dd["D"], dd["cu_seqlens"],
                                  None if init is None else init.cuda(), Q=Q)
    torch.cuda.synchronize()
    return y, fs


@pytest.mark.parametrize("path", PATHS, ids=[p[0] for p in PATHS])
@pytest.mark.parametrize("mix", list(MIXES))
@pytest.mark.parametrize("with_init", [False, True])
def test_varlen_matches_oracle(oracle, path, mix, with_init):
    name, H, P, G, N, Q, dtype = path
    lengths = MIXES[mix]
    d = synth.make_varlen(lengths, H, P, G, N, dtype, seed=700 + len(lengths))
    init = synth.make_state(len(lengths), H, P, N, seed=701, scale=0.5) if with_init else None
    announce("varlen", name, mix, with_init)
    y, fs = _run(d, Q, init)
    y_ref, fs_ref = oracle.ssd_scan_varlen(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["cu_seqlens"], d["D"],
                                           init)
    assert rel_err(y, y_ref) <= _tol(dtype)
    assert rel_err(fs, fs_ref) <= _tol(dtype)
    if init is not None:
        for b, n in enumerate(lengths):
            if n == 0:
                assert torch.equal(fs[b].cpu(), init[b])


@pytest.mark.parametrize("path", PATHS[:2], ids=[p[0] for p in PATHS[:2]])
def test_varlen_equal_lengths_bitwise_equals_batched(path):
    """Equal lengths: the same chunks as the batched call, the same bits."""
    name, H, P, G, N, Q, dtype = path
    B, L = 3, 520
    d = synth.make_prefill(B, L, H, P, G, N, dtype, seed=702)
    init = synth.make_state(B, H, P, N, seed=703, scale=0.5).cuda()
    dd = dev(d)
    announce("varlen equal lengths", name)
    y_b, fs_b = bd.ssd_prefill(dd["x"], dd["dt"], dd["A_log"], dd["Bm"], dd["Cm"], dd["D"], init, Q=Q)
    cu = torch.arange(0, (B + 1) * L, L, dtype=torch.int32, device="cuda")
    y_v, fs_v = bd.ssd_prefill_varlen(dd["x"].reshape(B * L, H, P), dd["dt"].reshape(B * L, H), dd["A_log"],
                                      dd["Bm"].reshape(B * L, G, N), dd["Cm"].reshape(B * L, G, N), dd["D"], cu,
                                      init, Q=Q)
    torch.cuda.synchronize()
    assert torch.equal(y_v, y_b.reshape(B * L, H, P))
    assert torch.equal(fs_v, fs_b)


def test_varlen_all_empty_keeps_states():
    H, P, G, N = 2, 64, 1, 128
    init = synth.make_state(3, H, P, N, seed=704).cuda()
    x = torch.empty((0, H, P), dtype=torch.bfloat16, device="cuda")
    bc = torch.empty((0, G, N), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(4, dtype=torch.int32, device="cuda")
    announce("varlen all empty")
    _, fs = bd.ssd_prefill_varlen(x, torch.empty((0, H), device="cuda"), torch.zeros(H, device="cuda"), bc, bc,
                                  None, cu, init, Q=256)
    torch.cuda.synchronize()
    assert torch.equal(fs, init)


@pytest.mark.parametrize("path", PATHS[:2], ids=[p[0] for p in PATHS[:2]])
def test_varlen_more_sequences_than_one_table_pass(oracle, path):
    """1500 sequences (the chunk table is laid out 1024 sequences per pass),
    lengths log-uniform in [1, 300], checked on sampled sequences."""
    name, H, P, G, N, Q, dtype = path
    lengths = synth.make_lengths(1500, 1, 300, seed=705)
    d = synth.make_varlen(lengths, H, P, G, N, dtype, seed=706)
    announce("varlen 1500 sequences", name)
    y, fs = _run(d, Q)
    cu = d["cu_seqlens"].numpy()
    for b in [0, 1, 511, 1023, 1024, 1025, 1499]:
        lo, hi = int(cu[b]), int(cu[b + 1])
        sub = dict(x=d["x"][None, lo:hi], dt=d["dt"][None, lo:hi], A_log=d["A_log"], Bm=d["Bm"][None, lo:hi],
                   Cm=d["Cm"][None, lo:hi], D=d["D"])
        y_ref, fs_ref = oracle.ssd_scan(**sub)
        assert rel_err(y[lo:hi], y_ref[0]) <= _tol(dtype), b
        assert rel_err(fs[b:b + 1], fs_ref) <= _tol(dtype), b


def test_varlen_serving_mix_sampled(oracle):
    """16 prompts of the 2.7B-shaped layer, lengths log-uniform in [64, 4096]
    (the bench's varlen workload), checked on sampled (sequence, head) pairs."""
    H, P, G, N = 80, 64, 1, 128
    lengths = synth.make_lengths(16, 64, 4096, seed=9)
    d = synth.make_varlen(lengths, H, P, G, N, "bf16", seed=10)
    announce("varlen serving mix", sum(lengths))
    y, fs = _run(d, 256)
    cu = d["cu_seqlens"].numpy()
    for b, h in [(0, 0), (5, 33), (15, 79)]:
        lo, hi = int(cu[b]), int(cu[b + 1])
        sub = dict(x=d["x"][None, lo:hi, h:h + 1], dt=d["dt"][None, lo:hi, h:h + 1], A_log=d["A_log"][h:h + 1],
                   Bm=d["Bm"][None, lo:hi], Cm=d["Cm"][None, lo:hi], D=d["D"][h:h + 1])
        y_ref, fs_ref = oracle.ssd_scan(**sub)
        assert rel_err(y[lo:hi, h:h + 1], y_ref[0]) <= TOL_BF16, (b, h)
        assert rel_err(fs[b:b + 1, h:h + 1], fs_ref) <= TOL_BF16, (b, h)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("K", [2, 4, 8])
@pytest.mark.parametrize("mix", list(MIXES))
def test_conv_varlen_matches_oracle(oracle, dtype, K, mix):
    """Depthwise conv over packed sequences: outputs and per-sequence caches
    (sequences shorter than K-1 keep part of their old cache; empty ones keep
    all of it)."""
    lengths = MIXES[mix] + [2]
    C = 96
    x = synth.make_tokens(1, sum(lengths), C, dtype, seed=720 + K)[0]
    w, bias = synth.make_conv(C, K, dtype, seed=721, with_bias=True)
    st = synth.make_tokens(len(lengths), K - 1, C, dtype, seed=722).transpose(1, 2).contiguous()
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    stg = st.cuda()
    announce("conv varlen", dtype, K, mix)
    out = bd.conv_state_update_varlen(stg, x.cuda(), cu.cuda(), w.cuda(), bias.cuda(), activation=1)
    torch.cuda.synchronize()
    new_ref, out_ref = oracle.conv_update_varlen(st, x, cu, w, bias, True)
    np.testing.assert_array_equal(stg.cpu().double().numpy(), new_ref)   # raw values, shifted exactly
    assert rel_err(out, out_ref) <= (1e-6 if dtype == "f32" else 8e-3)


def test_conv_varlen_equal_lengths_bitwise_equals_batched():
    B, L, C, K = 3, 70, 5376, 4
    x = synth.make_tokens(B, L, C, "bf16", seed=723)
    w, _ = synth.make_conv(C, K, "bf16", seed=724)
    st = synth.make_tokens(B, K - 1, C, "bf16", seed=725).transpose(1, 2).contiguous()
    s1, s2 = st.cuda(), st.cuda()
    announce("conv varlen equal lengths")
    o1 = bd.conv_state_update(s1, x.cuda(), w.cuda(), activation=1)
    cu = torch.arange(0, (B + 1) * L, L, dtype=torch.int32, device="cuda")
    o2 = bd.conv_state_update_varlen(s2, x.reshape(B * L, C).cuda(), cu, w.cuda(), activation=1)
    torch.cuda.synchronize()
    assert torch.equal(o2, o1.reshape(B * L, C))
    assert torch.equal(s2, s1)


def test_packed_prompts_then_decode(oracle):
    """Serving path on packed prompts: conv and SSD prefill over the packed
    batch, then one cached decode step per sequence from the caches they
    left, against the oracle's per-sequence run over prompt + 1 tokens."""
    H, P, G, N, K = 4, 64, 1, 128, 4
    lengths = [300, 1, 0, 513]
    C = H * P + 2 * G * N
    T = sum(lengths)
    xbc = synth.make_tokens(1, T + len(lengths), C, "bf16", seed=730)[0]
    prompt, step_tok = xbc[:T], xbc[T:]
    dts = synth.make_decode_stream(1, len(lengths), H, P, G, N, "bf16", seed=731)[1][0]
    d = synth.make_varlen(lengths, H, P, G, N, "bf16", seed=732)
    w, bias = synth.make_conv(C, K, "bf16", seed=733, with_bias=True)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
    conv0 = torch.zeros((len(lengths), C, K - 1), dtype=torch.bfloat16)
    announce("packed prompts then decode")
    cst = conv0.cuda()
    xc = bd.conv_state_update_varlen(cst, prompt.cuda(), cu.cuda(), w.cuda(), bias.cuda(), activation=1)
    x_p = xc[:, :H * P].reshape(T, H, P).contiguous()
    B_p = xc[:, H * P:H * P + G * N].reshape(T, G, N).contiguous()
    C_p = xc[:, H * P + G * N:].reshape(T, G, N).contiguous()
    dd = dev(d)
    _, state = bd.ssd_prefill_varlen(x_p, dd["dt"], dd["A_log"], B_p, C_p, dd["D"], cu.cuda(), Q=256)
    row = step_tok.cuda()
    cout = torch.empty_like(cst)
    y = bd.ssd_decode_step(row[:, :H * P], dts.cuda(), dd["A_log"], row[:, H * P:H * P + G * N],
                           row[:, H * P + G * N:], dd["D"], state, in_stride=C, G=G, conv_state_in=cst,
                           conv_state_out=cout, conv_w=w.cuda(), conv_b=bias.cuda(), K=K, activation=1)
    torch.cuda.synchronize()
    # oracle: per sequence, conv over the prompt then the scan, then one step
    new_c, xc_ref = oracle.conv_update_varlen(conv0, prompt, cu, w, bias, True)
    _, st_ref = oracle.ssd_scan_varlen(xc_ref[:, :H * P].reshape(T, H, P), d["dt"], d["A_log"],
                                       xc_ref[:, H * P:H * P + G * N].reshape(T, G, N),
                                       xc_ref[:, H * P + G * N:].reshape(T, G, N), cu, d["D"])
    r = step_tok
    y_ref, st2, _ = oracle.decode_step(r[:, :H * P], dts, d["A_log"], r[:, H * P:H * P + G * N],
                                       r[:, H * P + G * N:], d["D"], st_ref, conv_state=new_c, conv_w=w,
                                       conv_b=bias, activation=True)
    assert rel_err(y, y_ref) <= TOL_BF16
    assert rel_err(state, st2) <= TOL_BF16


@pytest.mark.parametrize("path", PATHS[:2], ids=[p[0] for p in PATHS[:2]])
def test_varlen_dt_raw_matches_oracle(oracle, path):
    """Packed sequences with the step preprocessed in the kernels."""
    name, H, P, G, N, Q, dtype = path
    lengths = MIXES["edges"]
    d = synth.make_varlen(lengths, H, P, G, N, dtype, seed=740)
    raw, dt_bias = synth.make_dt_raw((sum(lengths),), H, seed=741)
    init = synth.make_state(len(lengths), H, P, N, seed=742, scale=0.5)
    dd = dev(d)
    announce("varlen dt_raw", name)
    y, fs = bd.ssd_prefill_varlen(dd["x"], raw.cuda(), dd["A_log"], dd["Bm"], dd["Cm"], dd["D"], dd["cu_seqlens"],
                                  init.cuda(), Q=Q, dt_raw=True, dt_bias=dt_bias.cuda(), dt_min=1e-3, dt_max=0.1)
    torch.cuda.synchronize()
    dt_ref = oracle.dt_from_raw(raw, dt_bias, 1e-3, 0.1)
    y_ref, fs_ref = oracle.ssd_scan_varlen(d["x"], dt_ref, d["A_log"], d["Bm"], d["Cm"], d["cu_seqlens"], d["D"], init)
    assert rel_err(y, y_ref) <= _tol(dtype)
    assert rel_err(fs, fs_ref) <= _tol(dtype)
