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
    ("vector-bf16-q512", 2, 64, 1, 128, 512, "bf16"),
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
