"""Pins that tie the CPU oracle to the pages and to mathematics (CPU only).

Each check is computed by a route other than the oracle's token loop, so that a
dropped term, a wrong sign or index, or a transposed operand in the oracle
fails at least one of them:
  * hand-derived examples under tests/golden/ (decay 1 and decay 1/2);
  * the quadratic (masked-matrix) dual form, built from an explicit segsum;
  * closed forms: A -> 0 running sums, a single token (rank-1 state), pure
    decay from an initial state;
  * a textbook special case: P = N = 1 with constant dt, B, C is a first-order
    IIR filter (scipy.signal.lfilter);
  * chunk-size invariance (segmented runs, and the numpy chunked form);
  * prefill-then-decode equals one longer prefill;
  * linearity, causality, independence of heads/batch, group broadcasting;
  * convolution: one-hot taps, numpy.convolve, torch SiLU;
  * step-size chain: softplus(0) = ln 2, softplus(u) - softplus(-u) = u,
    400-digit decimal log(1 + e^u), the per-head bias index, clip bounds;
  * packed sequences: equal lengths reproduce the batched layout, an empty
    sequence keeps its state, sequences do not see each other;
  * gated RMS normalisation: torch's rms_norm and silu on the gated values,
    unit RMS per group, scale invariance, group independence, a constant
    group's closed form, a saturated gate.
"""
import decimal
import json
import math
import os

import numpy as np
import pytest
import scipy.signal
import torch

from mamba_ssd_scan_chunk_amd import synth
from tests.chunked_ref import chunked_ssd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _inputs(B=2, L=37, H=3, P=4, G=1, N=5, seed=0, variant="spec"):
    d = synth.make_prefill(B, L, H, P, G, N, "f32", seed, variant)
    return {k: v.numpy().astype(np.float64) for k, v in d.items()}


def _quadratic_form(x, dt, A_log, Bm, Cm, D, h0):
    """y_t = sum_{s<=t} (C_t . B_s) exp(sum_{r=s+1..t} a_r) dt_s x_s
             + exp(sum_{r<=t} a_r) C_t . h0 + D x_t
    with segsums written out as explicit loops (O(L^3), tiny inputs)."""
    Bsz, L, H, P = x.shape
    G, N = Bm.shape[2:]
    y = np.zeros_like(x)
    fs = np.zeros((Bsz, H, P, N))
    for b in range(Bsz):
        for h in range(H):
            g = h // (H // G)
            a = dt[b, :, h] * (-math.exp(A_log[h]))
            seg = np.full((L, L), -np.inf)
            for t in range(L):
                for s in range(t + 1):
                    seg[t, s] = sum(a[s + 1:t + 1])
            Lmat = np.exp(seg)  # lower triangular, zero above the diagonal
            CB = Cm[b, :, g, :] @ Bm[b, :, g, :].T
            M = CB * Lmat * dt[b, None, :, h]
            y[b, :, h, :] = M @ x[b, :, h, :]
            tot = np.array([sum(a[:t + 1]) for t in range(L)])
            y[b, :, h, :] += np.exp(tot)[:, None] * (Cm[b, :, g, :] @ h0[b, h].T)
            y[b, :, h, :] += D[h] * x[b, :, h, :]
            wend = np.exp(np.array([sum(a[s + 1:]) for s in range(L)])) * dt[b, :, h]
            fs[b, h] = math.exp(sum(a)) * h0[b, h] + np.einsum(
                "s,sp,sn->pn", wend, x[b, :, h, :], Bm[b, :, g, :])
    return y, fs


def test_golden_unit_decay(oracle):
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_unit_decay.json")))
    y, fs = oracle.ssd_scan(np.array(g["x"]), np.array(g["dt"]), np.array(g["A_log"]),
                            np.array(g["Bm"]), np.array(g["Cm"]), np.array(g["D"]))
    np.testing.assert_allclose(y, np.array(g["y"]), rtol=0, atol=1e-15)
    np.testing.assert_allclose(fs, np.array(g["final_state"]), rtol=0, atol=1e-15)


def test_golden_halving(oracle):
    g = json.load(open(os.path.join(GOLDEN, "hand_worked_halving.json")))
    ln2 = math.log(2.0)
    x = np.array(g["x"])
    dt = np.full(x.shape[:3], g["dt_ln2_multiple"] * ln2)
    y, fs = oracle.ssd_scan(x, dt, np.array(g["A_log"]), np.array(g["Bm"]),
                            np.array(g["Cm"]), np.array(g["D"]), np.array(g["init_state"]))
    yc = np.array(g["y_coeffs"])
    fc = np.array(g["final_state_coeffs"])
    np.testing.assert_allclose(y, yc[..., 0] + yc[..., 1] * ln2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(fs, fc[..., 0] + fc[..., 1] * ln2, rtol=0, atol=1e-13)


@pytest.mark.parametrize("G,H", [(1, 1), (1, 3), (3, 3), (2, 4)])
@pytest.mark.parametrize("with_h0", [False, True])
def test_quadratic_dual_form(oracle, G, H, with_h0):
    d = _inputs(B=2, L=29, H=H, P=3, G=G, N=4, seed=11 + G + H)
    h0 = synth.make_state(2, H, 3, 4, seed=5).numpy().astype(np.float64) if with_h0 else np.zeros((2, H, 3, 4))
    y, fs = oracle.ssd_scan(**d, init_state=h0 if with_h0 else None)
    yq, fq = _quadratic_form(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], h0)
    scale = np.abs(yq).max()
    assert np.abs(y - yq).max() <= 1e-12 * scale
    assert np.abs(fs - fq).max() <= 1e-12 * np.abs(fq).max()


def test_quadratic_dual_form_slow_decay(oracle):
    d = _inputs(B=1, L=64, H=2, P=8, G=1, N=8, seed=3, variant="slow")
    y, fs = oracle.ssd_scan(**d)
    yq, fq = _quadratic_form(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], np.zeros((1, 2, 8, 8)))
    assert np.abs(y - yq).max() <= 1e-12 * np.abs(yq).max()
    assert np.abs(fs - fq).max() <= 1e-12 * np.abs(fq).max()


def test_zero_A_is_running_sum(oracle):
    d = _inputs(B=2, L=40, H=2, P=3, G=1, N=4, seed=2)
    d["A_log"][:] = -200.0  # A = -exp(-200): exp(dt*A) == 1.0 exactly
    y, fs = oracle.ssd_scan(**d)
    xd = d["dt"][..., None] * d["x"]                        # [B,L,H,P]
    outer = xd[..., :, None] * d["Bm"][:, :, [0, 0], None, :]  # [B,L,H,P,N]
    S = np.cumsum(outer, axis=1)
    y_ref = np.einsum("blhpn,bln->blhp", S, d["Cm"][:, :, 0, :]) + d["D"][None, None, :, None] * d["x"]
    np.testing.assert_allclose(y, y_ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fs, S[:, -1], rtol=1e-12, atol=1e-12)


def test_single_token_rank_one(oracle):
    d = _inputs(B=1, L=1, H=2, P=6, G=1, N=5, seed=4)
    y, fs = oracle.ssd_scan(**d)
    for h in range(2):
        sv = np.linalg.svd(fs[0, h], compute_uv=False)
        assert sv[1] <= 1e-14 * sv[0]
        dt = d["dt"][0, 0, h]
        xv, Bv, Cv = d["x"][0, 0, h], d["Bm"][0, 0, 0], d["Cm"][0, 0, 0]
        np.testing.assert_allclose(fs[0, h], dt * np.outer(xv, Bv), rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(y[0, 0, h], dt * (Cv @ Bv) * xv + d["D"][h] * xv, rtol=1e-13, atol=1e-14)


def test_lti_first_order_iir_matches_lfilter(oracle):
    L = 300
    rng = np.random.default_rng(7)
    x = rng.standard_normal(L)
    dt, A_log, Bc, Cc, D = 0.07, math.log(3.0), 0.8, -1.3, 0.4
    pole = math.exp(dt * -math.exp(A_log))
    y, fs = oracle.ssd_scan(x.reshape(1, L, 1, 1), np.full((1, L, 1), dt), np.array([A_log]),
                            np.full((1, L, 1, 1), Bc), np.full((1, L, 1, 1), Cc), np.array([D]))
    ref = Cc * Bc * dt * scipy.signal.lfilter([1.0], [1.0, -pole], x) + D * x
    np.testing.assert_allclose(y.ravel(), ref, rtol=1e-11, atol=1e-12)


def test_pure_decay_from_initial_state(oracle):
    d = _inputs(B=1, L=50, H=3, P=4, G=1, N=3, seed=8)
    d["x"][:] = 0.0
    h0 = synth.make_state(1, 3, 4, 3, seed=9).numpy().astype(np.float64)
    y, fs = oracle.ssd_scan(**d, init_state=h0)
    A = -np.exp(d["A_log"])
    cum = np.cumsum(d["dt"][0] * A[None, :], axis=0)  # [L,H]
    np.testing.assert_allclose(fs[0], np.exp(cum[-1])[:, None, None] * h0[0], rtol=1e-12)
    y_ref = np.exp(cum)[:, :, None] * np.einsum("ln,hpn->lhp", d["Cm"][0, :, 0], h0[0])
    np.testing.assert_allclose(y[0], y_ref, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("Q", [1, 2, 3, 7, 16, 37])
def test_segmented_runs_equal_one_pass(oracle, Q):
    d = _inputs(B=2, L=37, H=3, P=4, G=1, N=5, seed=12)
    y, fs = oracle.ssd_scan(**d)
    state = None
    ys = []
    for c0 in range(0, 37, Q):
        sl = slice(c0, min(37, c0 + Q))
        yc, state = oracle.ssd_scan(d["x"][:, sl], d["dt"][:, sl], d["A_log"], d["Bm"][:, sl],
                                    d["Cm"][:, sl], d["D"], state)
        ys.append(yc)
    np.testing.assert_allclose(np.concatenate(ys, axis=1), y, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(state, fs, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("Q", [1, 4, 8, 16, 23, 64])
@pytest.mark.parametrize("variant", ["spec", "slow"])
def test_chunked_form_matches_oracle(oracle, Q, variant):
    d = _inputs(B=2, L=50, H=4, P=3, G=2, N=4, seed=13, variant=variant)
    h0 = synth.make_state(2, 4, 3, 4, seed=14).numpy().astype(np.float64)
    y, fs = oracle.ssd_scan(**d, init_state=h0)
    yc, hc = chunked_ssd(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], h0, Q=Q)
    assert np.abs(yc - y).max() <= 1e-12 * np.abs(y).max()
    assert np.abs(hc - fs).max() <= 1e-12 * np.abs(fs).max()


def test_prefill_then_decode_equals_longer_prefill(oracle):
    Bsz, L, k, H, P, G, N = 2, 30, 6, 2, 4, 1, 8
    d = _inputs(B=Bsz, L=L + k, H=H, P=P, G=G, N=N, seed=15)
    y_full, fs_full = oracle.ssd_scan(**d)
    _, state = oracle.ssd_scan(d["x"][:, :L], d["dt"][:, :L], d["A_log"], d["Bm"][:, :L],
                               d["Cm"][:, :L], d["D"])
    for t in range(L, L + k):
        y_t, state, _ = oracle.decode_step(
            d["x"][:, t].reshape(Bsz, H * P), d["dt"][:, t], d["A_log"],
            d["Bm"][:, t].reshape(Bsz, G * N), d["Cm"][:, t].reshape(Bsz, G * N), d["D"], state)
        np.testing.assert_allclose(y_t, y_full[:, t], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(state, fs_full, rtol=1e-13, atol=1e-13)


def test_linearity_in_x_and_initial_state(oracle):
    d1 = _inputs(seed=20)
    d2 = _inputs(seed=21)
    h1 = synth.make_state(2, 3, 4, 5, seed=22).numpy().astype(np.float64)
    h2 = synth.make_state(2, 3, 4, 5, seed=23).numpy().astype(np.float64)
    base = {k: d1[k] for k in ("dt", "A_log", "Bm", "Cm", "D")}
    a, b = 0.7, -1.9
    ya, fa = oracle.ssd_scan(d1["x"], **base, init_state=h1)
    yb, fb = oracle.ssd_scan(d2["x"], **base, init_state=h2)
    yab, fab = oracle.ssd_scan(a * d1["x"] + b * d2["x"], **base, init_state=a * h1 + b * h2)
    np.testing.assert_allclose(yab, a * ya + b * yb, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(fab, a * fa + b * fb, rtol=1e-12, atol=1e-12)


def test_causality(oracle):
    d = _inputs(seed=24)
    y, _ = oracle.ssd_scan(**d)
    t0 = 17
    d2 = {k: v.copy() for k, v in d.items()}
    d2["x"][:, t0] += 3.0
    d2["Bm"][:, t0 + 1] -= 1.0
    d2["dt"][:, t0 + 2] = 0.05
    y2, _ = oracle.ssd_scan(**d2)
    np.testing.assert_array_equal(y2[:, :t0], y[:, :t0])
    assert np.abs(y2[:, t0] - y[:, t0]).max() > 1e-3


def test_heads_and_batch_independent_and_permutable(oracle):
    d = _inputs(B=3, H=4, G=1, seed=25)
    y, fs = oracle.ssd_scan(**d)
    hp, bp = [2, 0, 3, 1], [1, 2, 0]
    dp = dict(x=d["x"][bp][:, :, hp], dt=d["dt"][bp][:, :, hp], A_log=d["A_log"][hp],
              Bm=d["Bm"][bp], Cm=d["Cm"][bp], D=d["D"][hp])
    y2, fs2 = oracle.ssd_scan(**dp)
    np.testing.assert_array_equal(y2, y[bp][:, :, hp])
    np.testing.assert_array_equal(fs2, fs[bp][:, hp])


def test_one_group_equals_replicated_groups(oracle):
    d = _inputs(B=2, H=4, G=1, seed=26)
    y, fs = oracle.ssd_scan(**d)
    rep = dict(d, Bm=np.repeat(d["Bm"], 4, axis=2), Cm=np.repeat(d["Cm"], 4, axis=2))
    y2, fs2 = oracle.ssd_scan(**rep)
    np.testing.assert_array_equal(y2, y)
    np.testing.assert_array_equal(fs2, fs)


def test_group_mapping_is_contiguous(oracle):
    # G=2, H=4: heads 0,1 read group 0; heads 2,3 read group 1.
    d = _inputs(B=1, H=4, G=2, seed=27)
    y, _ = oracle.ssd_scan(**d)
    for h in range(4):
        g = h // 2
        sub = dict(x=d["x"][:, :, [h]], dt=d["dt"][:, :, [h]], A_log=d["A_log"][[h]],
                   Bm=d["Bm"][:, :, [g]], Cm=d["Cm"][:, :, [g]], D=d["D"][[h]])
        yh, _ = oracle.ssd_scan(**sub)
        np.testing.assert_array_equal(yh[:, :, 0], y[:, :, h])


def test_empty_sequence_keeps_state(oracle):
    d = _inputs(B=1, L=0, H=2, P=3, G=1, N=4, seed=28)
    h0 = synth.make_state(1, 2, 3, 4, seed=29).numpy().astype(np.float64)
    y, fs = oracle.ssd_scan(**d, init_state=h0)
    assert y.shape == (1, 0, 2, 3)
    np.testing.assert_array_equal(fs, h0)


# ---------------------------------------------------------------- convolution

def test_conv_one_hot_taps_pin_orientation(oracle):
    Bsz, T, C, K = 2, 9, 5, 4
    u = synth.make_tokens(Bsz, T, C, "f32", seed=30).numpy().astype(np.float64)
    st0 = synth.make_tokens(Bsz, K - 1, C, "f32", seed=31).numpy().astype(np.float64).transpose(0, 2, 1).copy()
    w_id = np.zeros((C, K)); w_id[:, K - 1] = 1.0
    st, out = oracle.conv_update(st0, u, w_id)
    np.testing.assert_array_equal(out, u)                       # newest tap = identity
    np.testing.assert_array_equal(st, u[:, -(K - 1):].transpose(0, 2, 1))
    w_old = np.zeros((C, K)); w_old[:, 0] = 1.0
    _, out = oracle.conv_update(st0, u, w_old)                  # oldest tap = (K-1)-token delay
    hist = np.concatenate([st0.transpose(0, 2, 1), u], axis=1)  # [B, K-1+T, C]
    np.testing.assert_array_equal(out, hist[:, :T])


def test_conv_matches_numpy_convolve_and_silu(oracle):
    Bsz, T, C, K = 2, 40, 6, 4
    u = synth.make_tokens(Bsz, T, C, "f32", seed=32).numpy().astype(np.float64)
    w, bias = synth.make_conv(C, K, "f32", seed=33, with_bias=True)
    w, bias = w.numpy().astype(np.float64), bias.numpy().astype(np.float64)
    st0 = synth.make_tokens(Bsz, K - 1, C, "f32", seed=34).numpy().astype(np.float64).transpose(0, 2, 1).copy()
    for act in (False, True):
        st, out = oracle.conv_update(st0, u, w, bias, act)
        for b in range(Bsz):
            for c in range(C):
                seq = np.concatenate([st0[b, c], u[b, :, c]])
                full = np.convolve(seq, w[c, ::-1])[K - 1:K - 1 + T] + bias[c]
                if act:
                    full = torch.nn.functional.silu(torch.from_numpy(full)).numpy()
                np.testing.assert_allclose(out[b, :, c], full, rtol=1e-13, atol=1e-14)
        np.testing.assert_array_equal(st, u[:, -(K - 1):].transpose(0, 2, 1))


def test_conv_split_stream_equals_one_pass(oracle):
    Bsz, T, C, K = 1, 20, 4, 4
    u = synth.make_tokens(Bsz, T, C, "f32", seed=35).numpy().astype(np.float64)
    w, _ = synth.make_conv(C, K, "f32", seed=36)
    w = w.numpy().astype(np.float64)
    st0 = np.zeros((Bsz, C, K - 1))
    st, out = oracle.conv_update(st0, u, w, None, True)
    s = st0
    outs = []
    for t in range(T):  # token by token, as a decode loop would
        s, o = oracle.conv_update(s, u[:, t:t + 1], w, None, True)
        outs.append(o)
    np.testing.assert_array_equal(np.concatenate(outs, axis=1), out)
    np.testing.assert_array_equal(s, st)


def test_conv_short_sequence_keeps_old_taps(oracle):
    Bsz, T, C, K = 1, 2, 3, 4  # T < K-1: one old tap survives
    u = synth.make_tokens(Bsz, T, C, "f32", seed=37).numpy().astype(np.float64)
    st0 = synth.make_tokens(Bsz, K - 1, C, "f32", seed=38).numpy().astype(np.float64).transpose(0, 2, 1).copy()
    w, _ = synth.make_conv(C, K, "f32", seed=39)
    st, _ = oracle.conv_update(st0, u, w.numpy())
    np.testing.assert_array_equal(st[:, :, 0], st0[:, :, 2])
    np.testing.assert_array_equal(st[:, :, 1:], u.transpose(0, 2, 1))


def test_decode_with_conv_matches_conv_then_scan(oracle):
    Bsz, H, P, G, N, K = 2, 2, 4, 1, 8, 4
    C = H * P + 2 * G * N
    xbc, dts = synth.make_decode_stream(3, Bsz, H, P, G, N, "f32", seed=40)
    xbc, dts = xbc.numpy().astype(np.float64), dts.numpy().astype(np.float64)
    w, _ = synth.make_conv(C, K, "f32", seed=41)
    w = w.numpy().astype(np.float64)
    d = _inputs(B=Bsz, L=1, H=H, P=P, G=G, N=N, seed=42)
    state = synth.make_state(Bsz, H, P, N, seed=43).numpy().astype(np.float64)
    cst = np.zeros((Bsz, C, K - 1))
    # reference: conv over the 3 tokens at once, then the scan over 3 tokens
    _, conv_out = oracle.conv_update(cst, xbc.transpose(1, 0, 2), w, None, True)
    xs = conv_out[:, :, :H * P].reshape(Bsz, 3, H, P)
    Bs = conv_out[:, :, H * P:H * P + G * N].reshape(Bsz, 3, G, N)
    Cs = conv_out[:, :, H * P + G * N:].reshape(Bsz, 3, G, N)
    y_ref, fs_ref = oracle.ssd_scan(xs, dts.transpose(1, 0, 2), d["A_log"], Bs, Cs, d["D"], state)
    st = state
    for t in range(3):
        y, st, cst = oracle.decode_step(xbc[t, :, :H * P], dts[t], d["A_log"], xbc[t, :, H * P:H * P + G * N],
                                        xbc[t, :, H * P + G * N:], d["D"], st, conv_state=cst, conv_w=w,
                                        activation=True)
        np.testing.assert_allclose(y, y_ref[:, t], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(st, fs_ref, rtol=1e-13, atol=1e-13)


def test_decode_cache_save_restore_continues_bit_for_bit(oracle):
    """The O(1) cache (ssm_state, conv_state) is the whole state of a
    generation (bqwf.cn article §2.1-§2.2): written out as bytes after k
    steps, read back and continued for m steps, the oracle gives the outputs
    and the final cache of the uninterrupted k + m steps bit for bit -- the
    same check the GPU decode runs, on the CPU."""
    Bsz, H, P, G, N, K, k, m = 2, 3, 4, 1, 8, 4, 5, 6
    C = H * P + 2 * G * N
    xbc, dts = synth.make_decode_stream(k + m, Bsz, H, P, G, N, "f32", seed=46)
    xbc, dts = xbc.numpy().astype(np.float64), dts.numpy().astype(np.float64)
    w, _ = synth.make_conv(C, K, "f32", seed=47)
    w = w.numpy().astype(np.float64)
    d = _inputs(B=Bsz, L=1, H=H, P=P, G=G, N=N, seed=48)

    def steps(st, cst, t0, t1):
        ys = []
        for t in range(t0, t1):
            y, st, cst = oracle.decode_step(xbc[t, :, :H * P], dts[t], d["A_log"], xbc[t, :, H * P:H * P + G * N],
                                            xbc[t, :, H * P + G * N:], d["D"], st, conv_state=cst, conv_w=w,
                                            activation=True)
            ys.append(y)
        return ys, st, cst

    st0 = synth.make_state(Bsz, H, P, N, seed=49).numpy().astype(np.float64)
    cst0 = synth.make_conv(C, K, "f32", seed=50)[0].numpy().astype(np.float64)[None, :, :K - 1].repeat(Bsz, 0)
    ys_a, st_a, cst_a = steps(st0, cst0, 0, k + m)
    ys_b, st_b, cst_b = steps(st0, cst0, 0, k)
    blob = (st_b.tobytes(), cst_b.tobytes())  # the whole cache, as bytes
    st_r = np.frombuffer(blob[0], dtype=np.float64).reshape(st_b.shape).copy()
    cst_r = np.frombuffer(blob[1], dtype=np.float64).reshape(cst_b.shape).copy()
    ys_c, st_c, cst_c = steps(st_r, cst_r, k, k + m)
    assert all(np.array_equal(a, b) for a, b in zip(ys_a, ys_b + ys_c))
    assert np.array_equal(st_a, st_c) and np.array_equal(cst_a, cst_c)
    # the cache is not a function of fewer steps: a perturbed restore diverges
    st_r[0, 0, 0, 0] += 1.0
    ys_d, _, _ = steps(st_r, cst_r, k, k + m)
    assert not np.array_equal(ys_d[0], ys_c[0])


def test_oracle_rejects_bad_groups(oracle):
    d = _inputs(B=1, L=4, H=3, P=2, G=2, N=2, seed=44)  # G does not divide H
    with pytest.raises(ValueError):
        oracle.ssd_scan(**d)


# ---------------------------------------------------------------------------
# Step-size chain dt = clip(softplus(dt_raw + dt_bias[h]), dt_min, dt_max)
# ---------------------------------------------------------------------------

def _softplus_decimal(u):
    """log(1 + e^u) in 400-digit decimal arithmetic (independent of libm; enough
    digits that 1 + e^u keeps e^u down to u = -700)."""
    with decimal.localcontext() as ctx:
        ctx.prec = 400
        return float((decimal.Decimal(u).exp() + 1).ln())


def test_dt_softplus_at_zero_is_ln2(oracle):
    assert oracle.dt_from_raw(np.zeros((1, 1)))[0, 0] == pytest.approx(math.log(2.0), rel=1e-15)


def test_dt_softplus_matches_decimal_and_odd_part_identity(oracle):
    u = np.concatenate([np.linspace(-40.0, 40.0, 161), [-700.0, -1e-8, 1e-8, 700.0]])
    sp = oracle.dt_from_raw(u[:, None])[:, 0]
    ref = np.array([_softplus_decimal(v) for v in u])
    np.testing.assert_allclose(sp, ref, rtol=2e-15, atol=0.0)
    sp_neg = oracle.dt_from_raw(-u[:, None])[:, 0]
    np.testing.assert_allclose(sp - sp_neg, u, rtol=1e-14, atol=1e-15)   # softplus(u) - softplus(-u) = u
    assert np.all(sp > 0.0) and np.all(np.diff(sp[:161]) > 0.0)           # positive, increasing


def test_dt_bias_is_per_head_on_the_last_axis(oracle):
    H = 5
    bias = np.array([-3.0, -1.0, 0.0, 0.5, 2.0])
    raw = np.zeros((2, 3, H))
    raw[1, 2, :] = 1.0
    dt = oracle.dt_from_raw(raw, bias)
    for h in range(H):
        np.testing.assert_allclose(dt[0, 0, h], _softplus_decimal(bias[h]), rtol=2e-15)
        np.testing.assert_allclose(dt[1, 2, h], _softplus_decimal(bias[h] + 1.0), rtol=2e-15)


def test_dt_clip_bounds(oracle):
    u = np.array([[-800.0, -8.0, -4.0, -2.0, 0.0, 3.0, 800.0]])
    lo, hi = 1e-3, 0.1
    dt = oracle.dt_from_raw(u, None, lo, hi)[0]
    ref = np.clip([_softplus_decimal(v) if abs(v) < 100 else max(v, 0.0) for v in u[0]], lo, hi)
    np.testing.assert_allclose(dt, ref, rtol=2e-15, atol=0.0)
    assert dt[0] == lo and dt[-1] == hi and lo < dt[2] < hi
    # equal bounds pin every value; an inverted range is rejected
    np.testing.assert_array_equal(oracle.dt_from_raw(u, None, 0.05, 0.05), np.full_like(u, 0.05))
    with pytest.raises(ValueError):
        oracle.dt_from_raw(u, None, 0.2, 0.1)


# ---------------------------------------------------------------------------
# Gated RMS normalisation out = rmsnorm_group(y * silu(z)) * w
# ---------------------------------------------------------------------------

def _norm_inputs(rows=5, D=48, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((rows, D)), rng.standard_normal((rows, D)), rng.uniform(0.5, 1.5, D)


@pytest.mark.parametrize("group", [1, 8, 16, 48])
def test_gated_rmsnorm_matches_torch_rms_norm(oracle, group):
    y, z, w = _norm_inputs(seed=group)
    got = oracle.gated_rmsnorm(y, z, w, group=group, eps=1e-5)
    g = torch.from_numpy(y) * torch.nn.functional.silu(torch.from_numpy(z))
    rows, D = y.shape
    ref = torch.nn.functional.rms_norm(g.reshape(rows, D // group, group), (group,), eps=1e-5).reshape(rows, D)
    ref = (ref * torch.from_numpy(w)).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-14)


def test_gated_rmsnorm_unit_rms_and_scale_invariance(oracle):
    y, _, _ = _norm_inputs(seed=3)
    out = oracle.gated_rmsnorm(y, group=16, eps=0.0)
    blocks = out.reshape(5, 3, 16)
    np.testing.assert_allclose((blocks ** 2).mean(-1), 1.0, rtol=1e-14)
    ratio = blocks / y.reshape(5, 3, 16)                    # one positive factor per group
    np.testing.assert_allclose(ratio, ratio[..., :1] * np.ones(16), rtol=1e-13)
    assert np.all(ratio > 0)
    np.testing.assert_allclose(oracle.gated_rmsnorm(7.5 * y, group=16, eps=0.0), out, rtol=1e-13)
    np.testing.assert_allclose(oracle.gated_rmsnorm(-2.0 * y, group=16, eps=0.0), -out, rtol=1e-13)


def test_gated_rmsnorm_groups_are_independent(oracle):
    y, z, w = _norm_inputs(seed=4)
    out = oracle.gated_rmsnorm(y, z, w, group=16)
    y2 = y.copy()
    y2[:, 16:32] *= 3.0
    y2[:, 20] += 1.0
    out2 = oracle.gated_rmsnorm(y2, z, w, group=16)
    np.testing.assert_array_equal(out2[:, :16], out[:, :16])
    np.testing.assert_array_equal(out2[:, 32:], out[:, 32:])
    assert not np.allclose(out2[:, 16:32], out[:, 16:32])


def test_gated_rmsnorm_constant_group_closed_form(oracle):
    a, eps = 0.3, 0.01
    y = np.full((1, 8), a)
    w = np.arange(1.0, 9.0)
    out = oracle.gated_rmsnorm(y, None, w, group=8, eps=eps)
    np.testing.assert_allclose(out[0], a / math.sqrt(a * a + eps) * w, rtol=1e-15)


def test_gated_rmsnorm_gate(oracle):
    y, _, _ = _norm_inputs(seed=5)
    # z = 0 closes the gate: silu(0) = 0, so the output is 0 (eps > 0)
    np.testing.assert_array_equal(oracle.gated_rmsnorm(y, np.zeros_like(y), group=8), 0.0)
    # a saturated gate (silu(z) = z for large z) scales y by a constant, which
    # the normalisation removes
    np.testing.assert_allclose(oracle.gated_rmsnorm(y, np.full_like(y, 40.0), group=8, eps=0.0),
                               oracle.gated_rmsnorm(y, group=8, eps=0.0), rtol=1e-13)
    # the gate multiplies channel by channel: a gate of 2 on one channel only
    z = np.full_like(y, 40.0)
    z[:, 3] = 80.0
    y2 = y.copy()
    y2[:, 3] *= 2.0
    np.testing.assert_allclose(oracle.gated_rmsnorm(y, z, group=8, eps=0.0),
                               oracle.gated_rmsnorm(y2, group=8, eps=0.0), rtol=1e-13)
    with pytest.raises(ValueError):
        oracle.gated_rmsnorm(y, group=7)                      # groups must tile the channels


# ---------------------------------------------------------------------------
# Packed sequences (varlen)
# ---------------------------------------------------------------------------

def test_varlen_equal_lengths_is_the_batched_layout(oracle):
    B, L, H, P, G, N = 3, 20, 2, 3, 1, 4
    d = _inputs(B=B, L=L, H=H, P=P, G=G, N=N, seed=70)
    h0 = np.random.default_rng(71).standard_normal((B, H, P, N))
    y_ref, fs_ref = oracle.ssd_scan(**d, init_state=h0)
    packed = {k: (v.reshape((B * L,) + v.shape[2:]) if k in ("x", "dt", "Bm", "Cm") else v) for k, v in d.items()}
    y, fs = oracle.ssd_scan_varlen(cu_seqlens=[0, L, 2 * L, 3 * L], init_state=h0, **packed)
    np.testing.assert_array_equal(y, y_ref.reshape(B * L, H, P))
    np.testing.assert_array_equal(fs, fs_ref)


def test_varlen_sequences_are_independent_and_empty_ones_keep_state(oracle):
    H, P, G, N = 2, 3, 1, 4
    cu = [0, 7, 7, 19, 20]
    d = _inputs(B=1, L=20, H=H, P=P, G=G, N=N, seed=72)
    packed = {k: (v[0] if k in ("x", "dt", "Bm", "Cm") else v) for k, v in d.items()}
    h0 = np.random.default_rng(73).standard_normal((4, H, P, N))
    y, fs = oracle.ssd_scan_varlen(cu_seqlens=cu, init_state=h0, **packed)
    np.testing.assert_array_equal(fs[1], h0[1])                   # empty sequence
    # perturbing sequence 2's tokens leaves sequences 0 and 3 unchanged
    x2 = packed["x"].copy()
    x2[7:19] += 1.0
    y2, fs2 = oracle.ssd_scan_varlen(cu_seqlens=cu, init_state=h0, **{**packed, "x": x2})
    np.testing.assert_array_equal(y2[:7], y[:7])
    np.testing.assert_array_equal(y2[19:], y[19:])
    np.testing.assert_array_equal(fs2[[0, 1, 3]], fs[[0, 1, 3]])
    assert not np.allclose(y2[7:19], y[7:19])
    # a sequence starts from its own state, not from the previous sequence's
    # end: its first output is dt x (C.B) + D x + C.(decay h0[b]) x-free term
    t = 7
    A = -np.exp(packed["A_log"])
    for h in range(H):
        st = np.exp(packed["dt"][t, h] * A[h]) * h0[2, h] + packed["dt"][t, h] * np.outer(packed["x"][t, h],
                                                                                            packed["Bm"][t, 0])
        np.testing.assert_allclose(y[t, h], st @ packed["Cm"][t, 0] + packed["D"][h] * packed["x"][t, h],
                                   rtol=1e-13, atol=1e-13)


def test_conv_varlen_equal_lengths_is_the_batched_conv(oracle):
    B, L, C, K = 3, 9, 5, 4
    rng = np.random.default_rng(80)
    st = rng.standard_normal((B, C, K - 1))
    x = rng.standard_normal((B, L, C))
    w = rng.standard_normal((C, K))
    bias = rng.standard_normal(C)
    nb, ob = oracle.conv_update(st, x, w, bias, True)
    nv, ov = oracle.conv_update_varlen(st, x.reshape(B * L, C), [0, L, 2 * L, 3 * L], w, bias, True)
    np.testing.assert_array_equal(nv, nb)
    np.testing.assert_array_equal(ov, ob.reshape(B * L, C))


def test_conv_varlen_sequences_independent_and_empty_keeps_cache(oracle):
    C, K = 4, 4
    rng = np.random.default_rng(81)
    cu = [0, 2, 2, 11]
    st = rng.standard_normal((3, C, K - 1))
    x = rng.standard_normal((11, C))
    w = rng.standard_normal((C, K))
    nv, ov = oracle.conv_update_varlen(st, x, cu, w)
    np.testing.assert_array_equal(nv[1], st[1])                      # empty sequence
    # sequence 0 has 2 < K-1 tokens: the new cache keeps its oldest cached tap
    np.testing.assert_array_equal(nv[0][:, 0], st[0][:, 2])
    np.testing.assert_array_equal(nv[0][:, 1:], x[0:2].T)
    # sequence 2's first output sees its own cache, not sequence 0's tokens
    np.testing.assert_allclose(ov[2], (w[:, :K - 1] * st[2]).sum(1) + w[:, K - 1] * x[2], rtol=1e-15)
    x2 = x.copy()
    x2[0:2] += 1.0
    _, ov2 = oracle.conv_update_varlen(st, x2, cu, w)
    np.testing.assert_array_equal(ov2[2:], ov[2:])
