"""Host-side accounting of bench.py: algorithmic flops and bytes counted by
brute force on small shapes, the per-kernel split adding up to the whole, the
committed counter summaries being picked up, and the one-GPU contract."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _flops_brute(B, L, H, P, G, N, Q):
    """Multiply-adds of the chunked scan counted one product at a time (x2)."""
    total = 0
    for _ in range(B):
        for c0 in range(0, L, Q):
            q = min(Q, L - c0)
            pairs = sum(1 for l in range(q) for s in range(q) if s <= l)  # causal (l, s) pairs
            total += G * pairs * N * 2          # C_l . B_s once per group
            total += H * pairs * P * 2          # masked product times x
            total += H * q * N * P * 2          # chunk state
            total += H * q * N * P * 2          # C h_{c-1}
            total += H * P * N * 2              # state pass
    return total


@pytest.mark.parametrize("shape", [(1, 256, 2, 16, 1, 16, 64), (2, 100, 4, 8, 2, 8, 32), (1, 5, 1, 4, 1, 4, 8)])
def test_prefill_flops_match_brute_force(shape):
    assert bench.prefill_flops(*shape) == _flops_brute(*shape)


def test_prefill_and_decode_bytes():
    B, L, H, P, G, N = 1, 4096, 80, 64, 1, 128
    # x and y (bf16), dt (fp32), B and C (bf16), final state (fp32), A_log and D
    assert bench.prefill_bytes(B, L, H, P, G, N) == 2 * L * H * P * 2 + 4 * L * H + 2 * L * G * N * 2 + 4 * H * P * N + 8 * H
    C, K, Bd = H * P + 2 * G * N, 4, 16
    expect = (8 * Bd * H * P * N            # state read and written, fp32
              + 2 * Bd * C * (K - 1) * 2    # conv window in and out
              + Bd * C * 2 + 4 * Bd * H     # new token, dt
              + C * K * 2 + Bd * H * P * 2 + 8 * H)
    assert bench.decode_bytes(Bd, H, P, G, N, K) == expect
    assert expect == 85302912  # the per-step figure the decode leg reports at B = 16


@pytest.mark.parametrize("shape", [(1, 4096, 80, 64, 1, 128, 256), (8, 16384, 80, 64, 1, 128, 256),
                                   (2, 700, 6, 64, 3, 128, 256)])
def test_stage_flops_add_up_to_the_call(shape):
    four = ("chunk_pack_mfma", "chunk_state_mfma", "state_pass_bf16", "chunk_out_mfma")
    assert sum(bench.stage_work(k, *shape)[1] for k in four) == bench.prefill_flops(*shape)
    chained = ("chunk_pack_mfma", "chunk_chain_mfma")
    assert sum(bench.stage_work(k, *shape, chained=True)[1] for k in chained) == bench.prefill_flops(*shape)


def test_stage_bytes():
    shape = (1, 4096, 80, 64, 1, 128, 256)
    assert bench.stage_work("chunk_out_mfma", *shape)[0] == 108396544
    B, L, H, P, G, N, Q = 8, 16384, 80, 64, 1, 128, 256
    nch, x = L // Q, B * L * H * P * 2
    tiles = 36 * 32 * 32 * 2
    # x and y, dt; G^T, B and C operands of every (batch, chunk); the
    # carried state out and back in between chunks; the final state
    expect = 2 * x + 4 * B * L * H + B * nch * (tiles + 2 * Q * N * 2) + 2 * B * H * (nch - 1) * P * N * 4 \
        + B * H * P * N * 4
    assert bench.stage_work("chunk_chain_mfma", B, L, H, P, G, N, Q, chained=True)[0] == expect


@pytest.mark.parametrize("kernels", [("chunk_pack_mfma", "chunk_chain_mfma"),
                                     ("chunk_pack_mfma", "state_pass_bf16")])
def test_algorithmic_bytes_cover_the_call(kernels):
    """The compulsory bytes of the scan are those of the pack kernel (B, C)
    and of the kernel that streams x, y, dt and the state; in the four-kernel
    form x is counted by both the chunk-state and the output kernel."""
    shape = (8, 16384, 80, 64, 1, 128)
    B, L, H, P, G, N = shape
    total = sum(bench.section8d_bytes(k, *shape) for k in kernels)
    if kernels[1] == "state_pass_bf16":
        total += bench.section8d_bytes("chunk_out_mfma", *shape)
    assert total == bench.prefill_bytes(*shape)


def test_committed_counter_summaries_are_used():
    """The committed rocprofv3 summaries match the kernel sources (else
    bench.py reports null for them)."""
    assert bench.measured_traffic("chunk_chain_mfma", "mamba2-2.7b-longctx") is not None
    assert bench.measured_traffic("chunk_pack_mfma", "mamba2-2.7b-longctx") is not None
    assert bench.measured_traffic("decode_step_kernel", "mamba2-2.7b-decode-b16") is not None
    counted = bench.measured_mfma("mamba2-2.7b-longctx")
    assert counted["chunk_chain_mfma"] >= bench.stage_work("chunk_chain_mfma", 8, 16384, 80, 64, 1, 128, 256,
                                                           chained=True)[1]
    assert bench.measured_mfma("mamba2-130m-prefill") == {}


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
