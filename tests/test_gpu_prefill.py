"""GPU parity of ssd_prefill against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from mamba_ssd_scan_chunk_amd import binding as bd
from mamba_ssd_scan_chunk_amd import synth
from tests.gpu_utils import TOL_BF16, TOL_F32, announce, dev, f64, rel_err

pytestmark = pytest.mark.gpu


def _tol(dtype):
    return TOL_F32 if dtype == "f32" else TOL_BF16


def _run(d, Q, init=None, **kw):
    dd = dev(d)
    y, fs = bd.ssd_prefill(dd["x"], dd["dt"], dd["A_log"], dd["Bm"], dd["Cm"], dd["D"],
                           None if init is None else init.cuda(), Q=Q, **kw)
    torch.cuda.synchronize()
    return y, fs


CASES = [
    # name, B, L, H, P, G, N, Q, dtype
    ("ssd-f32-tiny", 1, 256, 2, 16, 1, 16, 64, "f32"),
    ("ragged", 2, 200, 3, 16, 1, 16, 64, "f32"),
    ("q16", 1, 100, 2, 16, 1, 16, 16, "f32"),
    ("q32-groups", 2, 130, 4, 8, 2, 32, 32, "f32"),
    ("odd-dims", 1, 77, 3, 3, 3, 5, 24, "f32"),
    ("one-token", 2, 1, 2, 16, 1, 16, 64, "f32"),
    ("q-eq-l", 1, 64, 2, 16, 1, 16, 64, "f32"),
    ("bf16-small", 1, 300, 4, 32, 1, 64, 32, "bf16"),
    ("bf16-q256-ragged", 1, 700, 2, 64, 1, 128, 256, "bf16"),
    ("bf16-q128", 2, 384, 3, 64, 1, 128, 128, "bf16"),
    ("bf16-q64-groups", 1, 333, 4, 64, 2, 128, 64, "bf16"),
    # MFMA path (P=64, N=128, Q=256): several groups and batch elements, an
    # item count that is not a multiple of 8 (the XCD-aware item order)
    ("bf16-mfma-groups", 2, 600, 4, 64, 2, 128, 256, "bf16"),
    ("bf16-mfma-b3g3", 3, 513, 6, 64, 3, 128, 256, "bf16"),
    # the largest P, N, Q the vector path takes, and the smallest Q
    ("f32-max-dims", 1, 300, 1, 256, 1, 256, 256, "f32"),
    ("bf16-max-dims", 1, 270, 1, 256, 1, 256, 256, "bf16"),
    ("f32-min-q", 1, 50, 2, 1, 1, 1, 16, "f32"),
    # chunks longer than 256 tokens: Q = 512 as suggested for long contexts
    # (MFMA shape: 256-token sub-chunks; other shapes: the vector path with
    # 512-token chunks), up to the largest chunk, with ragged thread shares
    ("bf16-q512", 1, 1300, 2, 64, 1, 128, 512, "bf16"),
    ("bf16-q768-mfma", 2, 1700, 3, 64, 1, 128, 768, "bf16"),
    ("bf16-q512-vector", 1, 1300, 2, 64, 1, 64, 512, "bf16"),
    ("f32-q1024", 1, 2200, 2, 16, 1, 16, 1024, "f32"),
    ("f32-q384-groups", 2, 900, 4, 8, 2, 32, 384, "f32"),
    ("f32-q1000-eq-l", 1, 1000, 1, 4, 1, 8, 1000, "f32"),
    # the chained single-pass MFMA path (B*H >= 192 chains): ragged last
    # chunk, several groups, one chunk per chain (no hand-off), 512-token
    # chunks as 256-token sub-chunks, a chain count that is not a multiple
    # of the eight XCD shares
    ("chain-b16h16", 16, 300, 16, 64, 1, 128, 256, "bf16"),
    ("chain-groups", 8, 600, 32, 64, 4, 128, 256, "bf16"),
    ("chain-one-chunk", 32, 200, 8, 64, 1, 128, 256, "bf16"),
    ("chain-q512", 4, 700, 64, 64, 1, 128, 512, "bf16"),
    ("chain-b9h29", 9, 777, 29, 64, 1, 128, 256, "bf16"),
    ("chain-b8h24-fewest", 8, 400, 24, 64, 1, 128, 256, "bf16"),  # 192 chains: the fewest that take it
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("variant", ["spec", "d0", "slow", "steep", "dtzero"])
@pytest.mark.parametrize("with_init", [False, True])
def test_prefill_matches_oracle(oracle, case, variant, with_init):
    name, B, L, H, P, G, N, Q, dtype = case
    d = synth.make_prefill(B, L, H, P, G, N, dtype, seed=100 + [c[0] for c in CASES].index(name), variant=variant)
    init = synth.make_state(B, H, P, N, seed=5, scale=0.5) if with_init else None
    announce("prefill", name, variant, with_init)
    y, fs = _run(d, Q, init)
    y_ref, fs_ref = oracle.ssd_scan(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], init)
    assert rel_err(y, y_ref) <= _tol(dtype)
    assert rel_err(fs, fs_ref) <= _tol(dtype)


RAW_DT_CASES = ["ragged", "q32-groups", "one-token", "odd-dims", "bf16-small", "bf16-q256-ragged",
                "bf16-mfma-b3g3", "chain-b9h29"]


@pytest.mark.parametrize("name", RAW_DT_CASES)
@pytest.mark.parametrize("raw_dt", [(True, 1e-3, 0.1), (False, 0.0, float("inf"))], ids=["bias-clip", "plain"])
def test_prefill_dt_raw_matches_oracle(oracle, name, raw_dt):
    """dt preprocessing fused into the prefill kernels (vector and MFMA
    paths, ragged last chunk): the oracle scans dt_from_raw of the same raw
    step."""
    case = next(c for c in CASES if c[0] == name)
    _, B, L, H, P, G, N, Q, dtype = case
    with_bias, lo, hi = raw_dt
    d = synth.make_prefill(B, L, H, P, G, N, dtype, seed=400 + RAW_DT_CASES.index(name))
    raw, dt_bias = synth.make_dt_raw((B, L), H, seed=450 + RAW_DT_CASES.index(name))
    dt_bias = dt_bias if with_bias else None
    init = synth.make_state(B, H, P, N, seed=6, scale=0.5)
    announce("prefill dt_raw", name, raw_dt)
    d["dt"] = raw
    y, fs = _run(d, Q, init, dt_raw=True, dt_bias=None if dt_bias is None else dt_bias.cuda(), dt_min=lo, dt_max=hi)
    dt_ref = oracle.dt_from_raw(raw, dt_bias, lo, hi)
    y_ref, fs_ref = oracle.ssd_scan(d["x"], dt_ref, d["A_log"], d["Bm"], d["Cm"], d["D"], init)
    assert rel_err(y, y_ref) <= _tol(dtype)
    assert rel_err(fs, fs_ref) <= _tol(dtype)


@pytest.mark.parametrize("B,H", [(2, 3), (8, 40)], ids=["four-kernel", "chained"])
def test_mfma_longer_chunks_are_256_token_sub_chunks(B, H):
    """On the MFMA shape a chunk of 512 or 1024 tokens runs as 256-token
    sub-chunks linked by the state hand-off: the same arithmetic as Q = 256,
    so the same bits."""
    d = dev(synth.make_prefill(B, 1500, H, 64, 1, 128, "bf16", seed=460))
    announce("mfma Q=512/1024 vs 256", B, H)
    y0, f0 = bd.ssd_prefill(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], Q=256)
    for Q in (512, 1024):
        y1, f1 = bd.ssd_prefill(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], Q=Q)
        torch.cuda.synchronize()
        assert torch.equal(y1, y0) and torch.equal(f1, f0), Q


@pytest.mark.parametrize("with_init", [False, True])
def test_prefill_empty_sequence(with_init):
    B, H, P, N = 2, 3, 16, 16
    init = synth.make_state(B, H, P, N, seed=1).cuda() if with_init else None
    x = torch.empty((B, 0, H, P), device="cuda")
    Bm = torch.empty((B, 0, 1, N), device="cuda")
    announce("prefill L=0", with_init)
    y, fs = bd.ssd_prefill(x, torch.empty((B, 0, H), device="cuda"), torch.zeros(H, device="cuda"), Bm, Bm,
                           None, init, Q=64, final_state=torch.full((B, H, P, N), 7.0, device="cuda"))
    torch.cuda.synchronize()
    if with_init:
        assert torch.equal(fs, init)
    else:
        assert torch.count_nonzero(fs) == 0


@pytest.mark.parametrize("dtype,B,L,H,P,N,Q", [
    ("f32", 1, 150, 2, 16, 16, 64),        # vector path
    ("bf16", 1, 700, 4, 64, 128, 256),     # four MFMA kernels
    ("bf16", 4, 700, 64, 64, 128, 256),    # chained single pass: chunk 0 reads, the last chunk writes
    ("bf16", 4, 200, 64, 64, 128, 256),    # chained, one chunk: one workgroup reads and writes
], ids=["vector", "mfma", "chain", "chain-one-chunk"])
def test_final_state_may_alias_init_state(oracle, dtype, B, L, H, P, N, Q):
    d = synth.make_prefill(B, L, H, P, 1, N, dtype, seed=3)
    init = synth.make_state(B, H, P, N, seed=4)
    dd = dev(d)
    announce("prefill alias", dtype, B, L, H)
    y_sep, fs_sep = bd.ssd_prefill(dd["x"], dd["dt"], dd["A_log"], dd["Bm"], dd["Cm"], dd["D"], init.cuda(), Q=Q)
    st = init.clone().cuda()
    y = bd.ssd_prefill(dd["x"], dd["dt"], dd["A_log"], dd["Bm"], dd["Cm"], dd["D"], st, Q=Q, final_state=st)[0]
    torch.cuda.synchronize()
    assert torch.equal(st, fs_sep) and torch.equal(y, y_sep)
    _, fs_ref = oracle.ssd_scan(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], init)
    assert rel_err(st, fs_ref) <= _tol(dtype)


@pytest.mark.parametrize("dtype,P,N,Q,B,H", [("f32", 16, 16, 64, 1, 4), ("bf16", 64, 128, 256, 1, 4),
                                            ("bf16", 64, 128, 256, 4, 80)])
def test_prefill_is_deterministic(dtype, P, N, Q, B, H):
    d = synth.make_prefill(B, 1000, H, P, 1, N, dtype, seed=9)
    announce("prefill determinism", dtype, B, H)
    y1, f1 = _run(d, Q)
    y2, f2 = _run(d, Q)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


@pytest.mark.parametrize("dtype,P,N,Q,B,H", [("f32", 16, 16, 64, 1, 3), ("bf16", 64, 128, 256, 1, 3),
                                            ("bf16", 64, 128, 256, 4, 64)])
def test_split_prefill_equals_one_prefill(oracle, dtype, P, N, Q, B, H):
    L1, L2 = 300, 213
    d = synth.make_prefill(B, L1 + L2, H, P, 1, N, dtype, seed=10, variant="slow")
    announce("split prefill", dtype)
    y, fs = _run(d, Q)
    first = {k: (v[:, :L1].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    second = {k: (v[:, L1:].contiguous() if v.dim() > 1 else v) for k, v in d.items()}
    y1, f1 = _run(first, Q)
    y2, f2 = _run(second, Q, init=f1.cpu())
    y_ref, fs_ref = oracle.ssd_scan(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"])
    assert rel_err(torch.cat([y1, y2], 1), y_ref) <= _tol(dtype)
    assert rel_err(f2, fs_ref) <= _tol(dtype)
    assert rel_err(torch.cat([y1, y2], 1), y) <= 2 * _tol(dtype)


@pytest.mark.parametrize("dtype,P,N,Q,B,H", [("f32", 16, 16, 64, 2, 4), ("bf16", 64, 128, 256, 2, 4),
                                            ("bf16", 64, 128, 256, 8, 32)])
def test_prefill_then_decode_equals_longer_prefill(oracle, dtype, P, N, Q, B, H):
    """prefill(L) then k decode steps gives the outputs and state of
    prefill(L + k)."""
    L, k, G = 520, 24, 1
    d = synth.make_prefill(B, L + k, H, P, G, N, dtype, seed=11)
    dd = dev(d)
    announce("prefill+decode", dtype)
    y_long, fs_long = bd.ssd_prefill(dd["x"], dd["dt"], dd["A_log"], dd["Bm"], dd["Cm"], dd["D"], Q=Q)
    head = {kk: (v[:, :L].contiguous() if v.dim() > 1 else v) for kk, v in dd.items()}
    _, state = bd.ssd_prefill(head["x"], head["dt"], head["A_log"], head["Bm"], head["Cm"], head["D"], Q=Q)
    ys = []
    for t in range(L, L + k):
        ys.append(bd.ssd_decode_step(dd["x"][:, t].reshape(B, H * P).contiguous(), dd["dt"][:, t].contiguous(),
                                     dd["A_log"], dd["Bm"][:, t].reshape(B, G * N).contiguous(),
                                     dd["Cm"][:, t].reshape(B, G * N).contiguous(), dd["D"], state))
    torch.cuda.synchronize()
    y_ref, fs_ref = oracle.ssd_scan(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"])
    y_dec = torch.stack(ys, 1)
    assert rel_err(y_dec, y_ref[:, L:]) <= _tol(dtype)
    assert rel_err(y_long[:, L:], y_ref[:, L:]) <= _tol(dtype)
    assert rel_err(state, fs_ref) <= _tol(dtype)
    assert rel_err(fs_long, fs_ref) <= _tol(dtype)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["mamba2-130m-prefill", "mamba2-2.7b-prefill"])
@pytest.mark.parametrize("variant", ["spec", "d0", "slow"])
def test_full_size_prefill_matches_oracle(oracle, name, variant):
    """Whole outputs of the 130M- and 2.7B-shaped layers (L=4096, Q=256)."""
    w = synth.WORKLOADS[name]
    d = synth.make_prefill(w.B, w.L, w.H, w.P, w.G, w.N, w.dtype, seed=1, variant=variant)
    announce("full prefill", name, variant)
    y, fs = _run(d, w.Q)
    y_ref, fs_ref = oracle.ssd_scan(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"])
    assert rel_err(y, y_ref) <= TOL_BF16
    assert rel_err(fs, fs_ref) <= TOL_BF16


@pytest.mark.slow
def test_full_size_prefill_dt_raw(oracle):
    """2.7B-shaped layer (L=4096, Q=256) with the step preprocessed in the
    kernels from a raw projection, a per-head bias and the bounds 1e-3, 0.1."""
    w = synth.WORKLOADS["mamba2-2.7b-prefill"]
    d = synth.make_prefill(w.B, w.L, w.H, w.P, w.G, w.N, w.dtype, seed=2)
    raw, dt_bias = synth.make_dt_raw((w.B, w.L), w.H, seed=3)
    announce("full prefill dt_raw")
    d["dt"] = raw
    y, fs = _run(d, w.Q, dt_raw=True, dt_bias=dt_bias.cuda(), dt_min=1e-3, dt_max=0.1)
    dt_ref = oracle.dt_from_raw(raw, dt_bias, 1e-3, 0.1)
    y_ref, fs_ref = oracle.ssd_scan(d["x"], dt_ref, d["A_log"], d["Bm"], d["Cm"], d["D"])
    assert rel_err(y, y_ref) <= TOL_BF16
    assert rel_err(fs, fs_ref) <= TOL_BF16


def _longctx_heads(b):
    """Sampled heads of batch element b: the first and the last head (the
    items at both ends of the contiguous item range each XCD is given start
    and end on them), and one more that moves with b."""
    return [0, 79, (13 * b + 5) % 80]


def _oracle_heads(oracle, d, b, heads, want_y=True):
    """The oracle's full scan of batch element b for a list of heads (one
    call, threads over the heads)."""
    idx = list(heads)
    return oracle.ssd_scan(d["x"][b:b + 1][:, :, idx], d["dt"][b:b + 1][:, :, idx], d["A_log"][idx],
                           d["Bm"][b:b + 1], d["Cm"][b:b + 1], d["D"][idx], want_y=want_y)


@pytest.mark.slow
def test_long_context_prefill_sampled_heads(oracle):
    """B=8, L=16384 2.7B-shaped layer: whole-run GPU outputs checked on three
    sampled heads of every batch element (24 (batch, head) pairs), each
    replayed by the oracle in full, and the final state of every head of the
    last batch element."""
    w = synth.WORKLOADS["mamba2-2.7b-longctx"]
    d = synth.make_prefill(w.B, w.L, w.H, w.P, w.G, w.N, w.dtype, seed=4)
    announce("longctx prefill")
    y, fs = _run(d, w.Q)
    y, fs = y.cpu(), fs.cpu()
    for b in range(w.B):
        heads = _longctx_heads(b)
        y_ref, fs_ref = _oracle_heads(oracle, d, b, heads)
        for j, h in enumerate(heads):
            assert rel_err(y[b, :, h], y_ref[0, :, j]) <= TOL_BF16, (b, h)
            assert rel_err(fs[b, h], fs_ref[0, j]) <= TOL_BF16, (b, h)
    b = w.B - 1
    _, fs_ref = _oracle_heads(oracle, d, b, range(w.H), want_y=False)
    assert rel_err(fs[b], fs_ref[0]) <= TOL_BF16


@pytest.mark.slow
def test_long_context_prefill_then_decode_sampled_heads(oracle):
    """B=8, L=16384 2.7B-shaped layer, then 1024 cached decode steps: the
    decode outputs and final state equal those of one prefill over all
    L + 1024 tokens, checked against the oracle's full scan on sampled
    (batch, head) pairs."""
    w = synth.WORKLOADS["mamba2-2.7b-longctx"]
    B, L, k, H, P, G, N = w.B, w.L, w.decode_steps, w.H, w.P, w.G, w.N
    d = synth.make_prefill(B, L + k, H, P, G, N, w.dtype, seed=5)
    announce("longctx prefill + decode", B, L, k)
    dd = dev(d)
    head = {kk: (v[:, :L].contiguous() if v.dim() > 1 else v) for kk, v in dd.items()}
    _, state = bd.ssd_prefill(head["x"], head["dt"], head["A_log"], head["Bm"], head["Cm"], head["D"], Q=w.Q)
    del head
    xs = dd["x"][:, L:].reshape(B, k, H * P).transpose(0, 1).contiguous()
    dts = dd["dt"][:, L:].transpose(0, 1).contiguous()
    Bs = dd["Bm"][:, L:].reshape(B, k, G * N).transpose(0, 1).contiguous()
    Cs = dd["Cm"][:, L:].reshape(B, k, G * N).transpose(0, 1).contiguous()
    y_dec = torch.empty((k, B, H, P), dtype=dd["x"].dtype, device="cuda")
    for t in range(k):
        bd.ssd_decode_step(xs[t], dts[t], dd["A_log"], Bs[t], Cs[t], dd["D"], state, y_t=y_dec[t], G=G)
    torch.cuda.synchronize()
    del dd
    y_dec, state = y_dec.cpu(), state.cpu()
    for b in range(B):
        heads = _longctx_heads(b + 3)
        y_ref, fs_ref = _oracle_heads(oracle, d, b, heads)
        for j, h in enumerate(heads):
            assert rel_err(y_dec[:, b, h], y_ref[0, L:, j]) <= TOL_BF16, (b, h)
            assert rel_err(state[b, h], fs_ref[0, j]) <= TOL_BF16, (b, h)


@pytest.mark.parametrize("dtype,P,N,Q,B,H,kernels", [
    ("bf16", 64, 128, 256, 1, 4, ["chunk_pack_mfma", "chunk_state_mfma", "state_pass_bf16", "chunk_out_mfma"]),
    ("bf16", 64, 128, 256, 4, 64, ["chunk_pack_mfma", "chunk_chain_mfma"]),
    ("f32", 16, 16, 64, 1, 4, ["chunk_state_vec", "chunk_cb_vec", "state_pass", "chunk_out_vec"]),
])
def test_stage_timing_reports_each_kernel(dtype, P, N, Q, B, H, kernels):
    d = synth.make_prefill(B, 700, H, P, 1, N, dtype, seed=12)
    announce("stage timing", dtype)
    y0, f0 = _run(d, Q)
    bd.stage_timing(True)
    try:
        y1, f1 = _run(d, Q)
        st = bd.stage_times()
    finally:
        bd.stage_timing(False)
    assert [name for name, _ in st] == kernels
    assert all(ms > 0.0 for _, ms in st)
    assert torch.equal(y0, y1) and torch.equal(f0, f1)  # timing changes no result


def test_stage_timing_is_per_host_thread():
    # two host threads time different paths at the same time; each reads back
    # only the kernels of its own last call
    import threading
    jobs = {
        "chain": (synth.make_prefill(4, 700, 64, 64, 1, 128, "bf16", seed=13),
                  ["chunk_pack_mfma", "chunk_chain_mfma"]),
        "four": (synth.make_prefill(1, 700, 4, 64, 1, 128, "bf16", seed=14),
                 ["chunk_pack_mfma", "chunk_state_mfma", "state_pass_bf16", "chunk_out_mfma"]),
    }
    announce("stage timing", "two threads")
    both = threading.Barrier(2)
    seen, errors = {}, []

    def work(key):
        try:
            d, _ = jobs[key]
            bd.stage_timing(True)
            try:
                _run(d, 256)
                both.wait(timeout=60)  # the other thread's call is enqueued too
                _run(d, 256)
                seen[key] = [name for name, _ in bd.stage_times()]
            finally:
                bd.stage_timing(False)
        except Exception as e:  # reported on the main thread
            errors.append(f"{key}: {e!r}")

    threads = [threading.Thread(target=work, args=(k,)) for k in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert errors == []
    assert {k: v for k, v in seen.items()} == {k: kernels for k, (_, kernels) in jobs.items()}


def test_expired_handoff_shows_as_nan_and_the_next_call_is_clean():
    # chained single pass (320 chains of 8 chunks); with a bound of 0 every
    # hand-off that does not find its predecessor already published expires,
    # which must show as NaN in that chain's state and outputs -- not hang --
    # and leave every other chain and the next call untouched
    B, L, H = 4, 2048, 80
    d = synth.make_prefill(B, L, H, 64, 1, 128, "bf16", seed=15)
    announce("hand-off expiry", f"B={B} L={L} H={H}")
    y0, f0 = _run(d, 256)
    assert torch.isfinite(f0).all() and torch.isfinite(y0.float()).all()
    bd.debug_handoff_ticks(0)
    try:
        y1, f1 = _run(d, 256)
    finally:
        bd.debug_handoff_ticks(-1)
    bad = torch.isnan(f1).flatten(2).any(-1)  # (B, H): chains with an expired wait
    assert bad.any()
    assert torch.isnan(y1.float().permute(0, 2, 1, 3)[bad]).any(-1).any(-1).all()
    good = ~bad
    assert torch.equal(f1[good], f0[good])
    assert torch.equal(y1.permute(0, 2, 1, 3)[good], y0.permute(0, 2, 1, 3)[good])
    y2, f2 = _run(d, 256)
    assert torch.equal(y2, y0) and torch.equal(f2, f0)


@pytest.mark.parametrize("B,L,H", [(4, 2048, 80), (9, 777, 29)])
def test_handoff_jitter_changes_no_result(B, L, H):
    # the chained single pass with random delays at every hand-off point: the
    # order in which workgroups start, wait and publish changes, the results
    # must not (they depend on no timing)
    d = synth.make_prefill(B, L, H, 64, 1, 128, "bf16", seed=16)
    init = synth.make_state(B, H, 64, 128, seed=17, scale=0.5)
    announce("hand-off jitter", f"B={B} L={L} H={H}")
    y0, f0 = _run(d, 256, init)
    for rounds in (40, 400):
        bd.debug_handoff_jitter(rounds)
        try:
            y1, f1 = _run(d, 256, init)
        finally:
            bd.debug_handoff_jitter(0)
        assert torch.equal(y1, y0) and torch.equal(f1, f0), rounds


def test_two_chained_prefills_on_two_streams_at_once():
    """Two chained single passes with their own workspaces run concurrently on
    two streams (default priority): each chain's hand-offs use only its own
    call's control block and slots, so both results equal their solo runs bit
    for bit."""
    shapes = [(4, 2048, 80, 20), (3, 1500, 64, 21)]  # 320 and 192 chains
    runs = []
    for B, L, H, seed in shapes:
        d = dev(synth.make_prefill(B, L, H, 64, 1, 128, "bf16", seed=seed))
        ws = torch.empty(bd.lib().ssd_prefill_workspace_bytes(B, L, H, 64, 1, 128, 256, bd.SSD_BF16),
                         dtype=torch.uint8, device="cuda")
        y = torch.empty_like(d["x"])
        fs = torch.empty((B, H, 64, 128), dtype=torch.float32, device="cuda")
        runs.append((d, ws, y, fs))

    def call(r, stream=None):
        d, ws, y, fs = r
        bd.ssd_prefill(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], Q=256, y=y, final_state=fs,
                       workspace=ws, stream=stream)

    announce("two chained prefills on two streams")
    solo = []
    for r in runs:
        call(r)
        torch.cuda.synchronize()
        solo.append((r[2].clone(), r[3].clone()))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        for r, s in zip(runs, streams):
            call(r, s)
    torch.cuda.synchronize()
    for (y0, f0), (_, _, y, fs) in zip(solo, runs):
        assert torch.equal(y, y0) and torch.equal(fs, f0)
