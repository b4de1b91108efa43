"""GPU parity of ssd_gated_rmsnorm (the layer's closing gated RMS
normalisation) against the CPU oracle, through the C ABI."""
import pytest
import torch

from mamba_ssd_scan_chunk_amd import binding as bd
from mamba_ssd_scan_chunk_amd import synth
from tests.gpu_utils import TOL_BF16, TOL_F32, announce, dev, rel_err

pytestmark = pytest.mark.gpu

# one bf16 rounding of an output of unit RMS; fp32 sums of up to 16k squares
TOL_NORM = {"bf16": 8e-3, "f32": 1e-5}

CASES = [
    # name, rows, D, group, dtype; fewer than 2048 rows: sixteen waves per row
    ("2.7b-whole-row", 300, 5120, 5120, "bf16"),     # 10 instructions per group
    ("130m-whole-row", 64, 1536, 1536, "bf16"),      # 3 of 4 instructions used
    ("per-head", 50, 5120, 64, "bf16"),              # 8 lanes per group
    ("group-512", 33, 4096, 512, "bf16"),            # one instruction per group
    ("group-1024", 9, 8192, 1024, "bf16"),           # runs of two instructions
    ("tiny-row", 7, 24, 8, "bf16"),                  # one vector per group, ragged instruction
    ("bf16-max", 5, 16384, 16384, "bf16"),           # 32 vectors per lane
    ("f32-2.7b-row", 40, 5120, 5120, "f32"),
    ("f32-group-256", 17, 1024, 256, "f32"),
    ("f32-group-4", 9, 64, 4, "f32"),
    ("f32-max", 3, 8192, 4096, "f32"),
    # 2048 rows or more: four waves per row instead of sixteen
    ("2.7b-prefill-rows", 2100, 5120, 5120, "bf16"),   # 3 vectors per thread, ragged
    ("per-head-many", 2048, 5120, 64, "bf16"),
    ("bf16-max-many", 2048, 16384, 2048, "bf16"),      # 8 vectors per thread, runs of 4 slots
    ("f32-many", 2050, 1024, 256, "f32"),
    ("f32-max-many", 2048, 8192, 8192, "f32"),         # one group of 32 slots
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("gated", [True, False])
@pytest.mark.parametrize("weighted", [True, False])
def test_gated_rmsnorm_matches_oracle(oracle, case, gated, weighted):
    name, rows, D, group, dtype = case
    seed = 600 + [c[0] for c in CASES].index(name)
    y = synth.make_tokens(1, rows, D, dtype, seed)[0]
    z, w = synth.make_gate((rows,), D, dtype, seed + 1)
    z, w = (z if gated else None), (w if weighted else None)
    announce("gated rmsnorm", name, gated, weighted)
    out = bd.ssd_gated_rmsnorm(y.cuda(), None if z is None else z.cuda(), None if w is None else w.cuda(),
                               group=group, eps=1e-5)
    torch.cuda.synchronize()
    ref = oracle.gated_rmsnorm(y, z, w, group=group, eps=1e-5)
    assert rel_err(out, ref) <= TOL_NORM[dtype]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gated_rmsnorm_strided_gate_and_in_place(oracle, dtype):
    """z as the first D columns of a wider projection [B, L, W]; out = y."""
    B, L, D, W = 2, 37, 1024, 1024 + 2 * 128 + 16
    y = synth.make_tokens(B, L, D, dtype, 1)
    proj, _ = synth.make_gate((B, L), W, dtype, 2)
    _, w = synth.make_gate((1,), D, dtype, 3)
    z = proj[..., :D]
    yd, zd = y.cuda(), proj.cuda()[..., :D]
    assert zd.stride() == (L * W, W, 1)
    announce("gated rmsnorm strided", dtype)
    out = bd.ssd_gated_rmsnorm(yd, zd, w.cuda(), group=512, eps=1e-6, out=yd)
    torch.cuda.synchronize()
    assert out.data_ptr() == yd.data_ptr()
    ref = oracle.gated_rmsnorm(y, z, w, group=512, eps=1e-6)
    assert rel_err(yd, ref) <= TOL_NORM[dtype]


def test_gated_rmsnorm_zero_gate_and_zero_rows():
    y = synth.make_tokens(1, 8, 512, "bf16", 3)[0].cuda()
    out = bd.ssd_gated_rmsnorm(y, torch.zeros_like(y), None, group=512, eps=1e-5)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
    empty = torch.empty((0, 512), dtype=torch.bfloat16, device="cuda")
    assert bd.ssd_gated_rmsnorm(empty, None, None, group=512).shape == (0, 512)


@pytest.mark.parametrize("dtype,P,N,Q", [("bf16", 64, 128, 256), ("f32", 16, 16, 64)])
def test_prefill_then_gated_norm_matches_oracle(oracle, dtype, P, N, Q):
    """The mixer's output side after a prefill: the scan's y [B, L, H*P],
    gated by z and normalised over all H*P channels (one group, as in the
    Mamba-2 2.7B layer), against the oracle's scan followed by its norm."""
    B, L, H, G = 2, 600, 4, 1
    d = synth.make_prefill(B, L, H, P, G, N, dtype, seed=31)
    z, w = synth.make_gate((B, L), H * P, dtype, seed=32)
    dd = dev(d)
    announce("prefill + gated norm", dtype)
    y, _ = bd.ssd_prefill(dd["x"], dd["dt"], dd["A_log"], dd["Bm"], dd["Cm"], dd["D"], Q=Q)
    out = bd.ssd_gated_rmsnorm(y.reshape(B, L, H * P), z.cuda(), w.cuda(), group=H * P, eps=1e-5)
    torch.cuda.synchronize()
    y_ref, _ = oracle.ssd_scan(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"])
    ref = oracle.gated_rmsnorm(y_ref.reshape(B, L, H * P), z, w, group=H * P, eps=1e-5)
    assert rel_err(out, ref) <= (TOL_F32 if dtype == "f32" else TOL_BF16)


def test_gated_rmsnorm_is_deterministic():
    y = synth.make_tokens(1, 256, 5120, "bf16", 5)[0].cuda()
    z, w = synth.make_gate((256,), 5120, "bf16", 6)
    announce("gated rmsnorm determinism")
    a = bd.ssd_gated_rmsnorm(y, z.cuda(), w.cuda(), group=5120)
    b = bd.ssd_gated_rmsnorm(y, z.cuda(), w.cuda(), group=5120)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
