"""GPU parity of ssd_prefill_varlen (sequences packed without padding)
against the CPU oracle, through the C ABI."""
import contextlib

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


# Packed sequences of the chained shape (bf16, P = 64, N = 128, a chunk
# length that is a multiple of 256, sequences x heads >= 192) launch both
# forms; the chunk-table kernel picks the chained pass when the effective
# chains H * (total chunks) / (most chunks of one sequence) reach 192, else
# the four-kernel form.  Each case runs both forms forced and the choice.
CHAIN_CASES = [
    # id, lengths, H, G
    ("edges-h64", MIXES["edges"], 64, 2),  # 64 * 9 / 3 = 192: chained, at the bound
    ("many-short-h32", MIXES["many-short"], 32, 2),
    ("one-h192", [600], 192, 2),
    ("balanced-long-h32", [1500, 1400, 1300, 1536, 0, 1200, 1100, 1000], 32, 2),
    ("long-and-short-h32", [5000, 3, 0, 1300, 256, 2049], 32, 4),  # 32 * 37 / 20: four-kernel
    ("one-dominates-h64", [6000, 100, 50, 0], 64, 2),
]
DUAL_STAGES = ["chunk_table_kernel", "chunk_pack_mfma", "chunk_chain_mfma", "chunk_state_mfma", "state_pass_bf16",
               "chunk_out_mfma"]


def _chained_by_lengths(lengths, H, Q=256):
    n = [(L + Q - 1) // Q for L in lengths]
    return max(n) > 0 and H * sum(n) >= 192 * max(n)


@contextlib.contextmanager
def packed_form(form):
    bd.debug_packed_form(form)
    try:
        yield
    finally:
        bd.debug_packed_form(-1)


def _run_staged(d, Q, init=None, final_state=None):
    """_run with stage timing on: (y, final_state, kernels that ran)."""
    dd = dev(d)
    bd.stage_timing(True)
    try:
        y, fs = bd.ssd_prefill_varlen(dd["x"], dd["dt"], dd["A_log"], dd["Bm"], dd["Cm"], dd["D"], dd["cu_seqlens"],
                                      init, Q=Q, final_state=final_state)
        torch.cuda.synchronize()
        st = [name for name, _ in bd.stage_times()]
    finally:
        bd.stage_timing(False)
    return y, fs, st


def test_chained_choice_by_lengths():
    assert [_chained_by_lengths(c[1], c[2]) for c in CHAIN_CASES] == [True, True, True, True, False, False]
    assert _chained_by_lengths(synth.make_lengths(16, 64, 4096, seed=9), 80)  # the serving mix


@pytest.mark.parametrize("case", CHAIN_CASES, ids=[c[0] for c in CHAIN_CASES])
@pytest.mark.parametrize("with_init", [False, True])
def test_varlen_chained_matches_oracle(oracle, case, with_init):
    name, lengths, H, G = case
    d = synth.make_varlen(lengths, H, 64, G, 128, "bf16", seed=750 + len(lengths))
    init = synth.make_state(len(lengths), H, 64, 128, seed=751, scale=0.5) if with_init else None
    y_ref, fs_ref = oracle.ssd_scan_varlen(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["cu_seqlens"], d["D"],
                                           init)
    out = {}
    for form in (1, 0, -1):
        announce("varlen chained", name, with_init, "form", form)
        with packed_form(form):
            y, fs, st = _run_staged(d, 256, None if init is None else init.cuda())
        assert st == DUAL_STAGES, form
        assert rel_err(y, y_ref) <= TOL_BF16, form
        assert rel_err(fs, fs_ref) <= TOL_BF16, form
        for b, n in enumerate(lengths):  # an empty sequence hands its state on unchanged
            if n == 0:
                want = init[b] if init is not None else torch.zeros_like(fs[b].cpu())
                assert torch.equal(fs[b].cpu(), want), form
        out[form] = (y, fs)
    chosen = out[1 if _chained_by_lengths(lengths, H) else 0]
    assert torch.equal(out[-1][0], chosen[0]) and torch.equal(out[-1][1], chosen[1])


@pytest.mark.parametrize("form", [1, 0])
def test_varlen_chained_final_state_may_alias_init_state(oracle, form):
    """final_state is init_state: the state of an empty sequence is copied
    onto itself; every other sequence reads its initial state before its
    last chunk writes the final one."""
    lengths = [700, 0, 1, 256, 0, 513]
    H = 48
    d = synth.make_varlen(lengths, H, 64, 1, 128, "bf16", seed=752)
    init = synth.make_state(len(lengths), H, 64, 128, seed=753, scale=0.5)
    announce("varlen chained alias", form)
    with packed_form(form):
        y_sep, fs_sep, st = _run_staged(d, 256, init.cuda())
        assert st == DUAL_STAGES
        buf = init.clone().cuda()
        y, _, _ = _run_staged(d, 256, buf, final_state=buf)
    assert torch.equal(buf, fs_sep) and torch.equal(y, y_sep)
    _, fs_ref = oracle.ssd_scan_varlen(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["cu_seqlens"], d["D"], init)
    assert rel_err(buf, fs_ref) <= TOL_BF16


EQUAL_PATHS = PATHS[:2] + [("chain", 64, 64, 2, 128, 256, "bf16")]


@pytest.mark.parametrize("path", EQUAL_PATHS, ids=[p[0] for p in EQUAL_PATHS])
def test_varlen_equal_lengths_bitwise_equals_batched(path):
    """Equal lengths: the same chunks as the batched call, the same bits (on
    the chained path, packed item order against the batched one)."""
    name, H, P, G, N, Q, dtype = path
    B, L = 4, 520
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


DT_RAW_PATHS = PATHS[:2] + [("chain", 64, 64, 2, 128, 256, "bf16")]  # edges at H = 64: 192 effective chains


@pytest.mark.parametrize("path", DT_RAW_PATHS, ids=[p[0] for p in DT_RAW_PATHS])
def test_varlen_dt_raw_matches_oracle(oracle, path):
    """Packed sequences with the step preprocessed in the kernels."""
    name, H, P, G, N, Q, dtype = path
    lengths = MIXES["edges"]
    assert name != "chain" or _chained_by_lengths(lengths, H)
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


JITTER_MIX = [1500, 1400, 0, 1300, 1536, 1200, 1100, 1000, 3]  # 32 * 39 / 6 = 208 chains: chained


def test_varlen_chained_handoff_jitter_changes_no_result():
    """The packed item order with random delays at every hand-off point: the
    order in which workgroups start, wait and publish changes, the results
    must not."""
    H = 32
    assert _chained_by_lengths(JITTER_MIX, H)
    d = synth.make_varlen(JITTER_MIX, H, 64, 2, 128, "bf16", seed=760)
    init = synth.make_state(len(JITTER_MIX), H, 64, 128, seed=761, scale=0.5).cuda()
    announce("varlen hand-off jitter")
    y0, f0, st = _run_staged(d, 256, init)
    assert st == DUAL_STAGES
    for rounds in (40, 400):
        bd.debug_handoff_jitter(rounds)
        try:
            y1, f1, _ = _run_staged(d, 256, init)
        finally:
            bd.debug_handoff_jitter(0)
        assert torch.equal(y1, y0) and torch.equal(f1, f0), rounds


def test_varlen_chained_expired_handoff_shows_as_nan_and_the_next_call_is_clean():
    """With a wait bound of 0, every hand-off that does not find its
    predecessor already published expires: NaN in that (sequence, head)
    chain, never a hang.  Sequences of one chunk (and empty ones) never wait,
    so their results are untouched, and the next call is clean."""
    H = 32
    d = synth.make_varlen(JITTER_MIX, H, 64, 2, 128, "bf16", seed=762)
    announce("varlen hand-off expiry")
    with packed_form(1):
        y0, f0, _ = _run_staged(d, 256)
        bd.debug_handoff_ticks(0)
        try:
            y1, f1, _ = _run_staged(d, 256)
        finally:
            bd.debug_handoff_ticks(-1)
        y2, f2, _ = _run_staged(d, 256)
    assert torch.isfinite(f0).all() and torch.isfinite(y0.float()).all()
    bad = torch.isnan(f1).flatten(2).any(-1)  # (sequence, head): chains with an expired wait
    assert bad.any()
    cu = d["cu_seqlens"].tolist()
    for b, n in enumerate(JITTER_MIX):
        rows = slice(cu[b], cu[b + 1])
        if n <= 256:  # one chunk or empty: nothing to wait for
            assert not bad[b].any()
            assert torch.equal(f1[b], f0[b]) and torch.equal(y1[rows], y0[rows])
        for h in range(H):
            if bad[b, h]:
                assert torch.isnan(y1[rows, h].float()).any()
            else:
                assert torch.equal(f1[b, h], f0[b, h]) and torch.equal(y1[rows, h], y0[rows, h])
    assert torch.equal(y2, y0) and torch.equal(f2, f0)


@pytest.mark.parametrize("form", [1, 0])
def test_varlen_every_short_chunk_tile_count(oracle, form):
    """One-chunk sequences of 1 to 8 token tiles, at both edges of each tile
    count: the output phase forms only the column tiles that hold a token of
    the chunk (a wave whose second tile is past the chunk forms its first
    alone), in both forms."""
    lengths = [1, 32, 33, 64, 65, 96, 97, 128, 129, 160, 161, 192, 193, 224, 225, 255, 256, 0]
    H = 16  # 16 * 17 / 1 effective chains: the chained pass when not forced
    d = synth.make_varlen(lengths, H, 64, 2, 128, "bf16", seed=770)
    init = synth.make_state(len(lengths), H, 64, 128, seed=771, scale=0.5)
    announce("varlen short chunk tiles", form)
    with packed_form(form):
        y, fs, st = _run_staged(d, 256, init.cuda())
    assert st == DUAL_STAGES
    y_ref, fs_ref = oracle.ssd_scan_varlen(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["cu_seqlens"], d["D"], init)
    assert rel_err(y, y_ref) <= TOL_BF16
    assert rel_err(fs, fs_ref) <= TOL_BF16
    cu = d["cu_seqlens"].tolist()
    for b in range(len(lengths)):  # every sequence on its own, not just the batch
        rows = slice(cu[b], cu[b + 1])
        if lengths[b]:
            assert rel_err(y[rows], y_ref[rows]) <= TOL_BF16, b
        assert rel_err(fs[b:b + 1], fs_ref[b:b + 1]) <= TOL_BF16, b


def test_varlen_many_short_prompts_sampled(oracle):
    """512 prompts of the 2.7B-shaped layer, 16-512 tokens each (the bench's
    many-short batch: most chunks short, the chained pass chosen), checked on
    sampled (sequence, head) pairs, including the first and last sequence."""
    H, P, G, N = 80, 64, 1, 128
    lengths = synth.make_lengths(512, 16, 512, seed=3)
    assert _chained_by_lengths(lengths, H)
    d = synth.make_varlen(lengths, H, P, G, N, "bf16", seed=10)
    announce("varlen many short", sum(lengths))
    y, fs = _run(d, 256)
    cu = d["cu_seqlens"].numpy()
    for b, h in [(0, 0), (1, 79), (137, 40), (255, 5), (256, 77), (400, 12), (510, 63), (511, 31)]:
        lo, hi = int(cu[b]), int(cu[b + 1])
        sub = dict(x=d["x"][None, lo:hi, h:h + 1], dt=d["dt"][None, lo:hi, h:h + 1], A_log=d["A_log"][h:h + 1],
                   Bm=d["Bm"][None, lo:hi], Cm=d["Cm"][None, lo:hi], D=d["D"][h:h + 1])
        y_ref, fs_ref = oracle.ssd_scan(**sub)
        assert rel_err(y[lo:hi, h:h + 1], y_ref[0]) <= TOL_BF16, (b, h)
        assert rel_err(fs[b:b + 1, h:h + 1], fs_ref) <= TOL_BF16, (b, h)


@pytest.mark.parametrize("long_chunks", [566, 567], ids=["lds", "scratch"])
def test_varlen_chained_at_the_table_lds_bound(oracle, long_chunks):
    """The chunk-table kernel's item-order histograms span the chunk counts up
    to the largest one: 18 * (566 + 2) ints = 40.9 KB is the most it keeps in
    LDS, one chunk more goes to global scratch.  One sequence of that many
    chunks and 15 short ones, the chained pass forced; sampled (sequence,
    head) pairs against the oracle."""
    H = 12  # 16 sequences x 12 heads = 192: both forms launched
    lengths = [256 * long_chunks - 100] + [300, 1, 0, 257, 64] * 3
    assert 18 * (566 + 2) * 4 <= 40 * 1024 < 18 * (567 + 2) * 4
    d = synth.make_varlen(lengths, H, 64, 1, 128, "bf16", seed=780)
    announce("varlen table LDS bound", long_chunks)
    with packed_form(1):
        y, fs, st = _run_staged(d, 256)
    assert st == DUAL_STAGES
    cu = d["cu_seqlens"].numpy()
    for b, h in [(0, 0), (0, 11), (1, 5), (4, 7)]:
        lo, hi = int(cu[b]), int(cu[b + 1])
        sub = dict(x=d["x"][None, lo:hi, h:h + 1], dt=d["dt"][None, lo:hi, h:h + 1], A_log=d["A_log"][h:h + 1],
                   Bm=d["Bm"][None, lo:hi], Cm=d["Cm"][None, lo:hi], D=d["D"][h:h + 1])
        y_ref, fs_ref = oracle.ssd_scan(**sub)
        assert rel_err(y[lo:hi, h:h + 1], y_ref[0]) <= TOL_BF16, (b, h)
        assert rel_err(fs[b:b + 1, h:h + 1], fs_ref) <= TOL_BF16, (b, h)


@pytest.mark.parametrize("seed", range(12))
def test_varlen_random_mixes(oracle, seed):
    """Seeded random packed batches of the chained shape: 1 to 40 sequences
    of 0 to 1500 tokens (some empty), 16 to 64 heads.  The chained pass
    (forced) matches the oracle, and the device's own choice gives the bits
    of the form the length rule names."""
    rng = np.random.default_rng(900 + seed)
    nseq = int(rng.integers(1, 41))
    H = int(rng.choice([16, 24, 32, 48, 64]))
    if nseq * H < 192:  # below the bound the call never launches the chained pass
        nseq = -(-192 // H)
    lengths = [int(v) for v in rng.integers(0, 1501, size=nseq)]
    lengths = [0 if rng.random() < 0.1 else n for n in lengths]
    if sum(lengths) == 0:
        lengths[0] = 1
    G = 2 if H % 2 == 0 else 1
    d = synth.make_varlen(lengths, H, 64, G, 128, "bf16", seed=901 + seed)
    init = synth.make_state(len(lengths), H, 64, 128, seed=902 + seed, scale=0.5)
    announce("varlen random mix", seed, nseq, H, sum(lengths))
    out = {}
    for form in (1, 0, -1):
        with packed_form(form):
            out[form] = _run_staged(d, 256, init.cuda())[:2]
    y_ref, fs_ref = oracle.ssd_scan_varlen(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["cu_seqlens"], d["D"],
                                           init)
    for form in (1, 0):
        assert rel_err(out[form][0], y_ref) <= TOL_BF16, form
        assert rel_err(out[form][1], fs_ref) <= TOL_BF16, form
    chosen = out[1 if _chained_by_lengths(lengths, H) else 0]
    assert torch.equal(out[-1][0], chosen[0]) and torch.equal(out[-1][1], chosen[1])


def test_varlen_packed_form_is_per_host_thread():
    """ssd_debug_packed_form is kept per host thread: two threads forcing
    different forms on the same packed batch at once (own streams, own
    outputs and workspaces) each get their own form's bits."""
    import threading

    lengths = [700, 0, 1, 256, 513, 90, 1200, 31]
    H = 32
    d = dev(synth.make_varlen(lengths, H, 64, 2, 128, "bf16", seed=790))
    T, B = sum(lengths), len(lengths)
    want = {}
    for form in (0, 1):
        with packed_form(form):
            y, fs = bd.ssd_prefill_varlen(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], d["cu_seqlens"],
                                          Q=256)
        torch.cuda.synchronize()
        want[form] = (y, fs)
    assert not torch.equal(want[0][0], want[1][0])  # the two forms round differently: the check can tell them apart
    announce("varlen packed form per thread")
    errors, got = [], {}

    def worker(form):
        try:
            bd.debug_packed_form(form)
            stream = torch.cuda.Stream()
            ws = torch.empty(bd.lib().ssd_prefill_varlen_workspace_bytes(B, T, H, 64, 2, 128, 256, bd.SSD_BF16),
                             dtype=torch.uint8, device="cuda")
            y = torch.empty_like(d["x"])
            fs = torch.empty((B, H, 64, 128), dtype=torch.float32, device="cuda")
            stream.wait_stream(torch.cuda.default_stream())
            with torch.cuda.stream(stream):
                for _ in range(5):
                    bd.ssd_prefill_varlen(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], d["cu_seqlens"],
                                          Q=256, y=y, final_state=fs, workspace=ws, stream=stream)
            stream.synchronize()
            got[form] = (y, fs)
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))
        finally:
            bd.debug_packed_form(-1)

    threads = [threading.Thread(target=worker, args=(f,)) for f in (0, 1)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert errors == []
    for form in (0, 1):
        assert torch.equal(got[form][0], want[form][0]) and torch.equal(got[form][1], want[form][1]), form
