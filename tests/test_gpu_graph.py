"""HIP-graph capture of the C-ABI calls (the on-device decode loop).

Each graph is captured once and replayed several times, with the program's
own eager work and synchronisations between replays; every replay must equal
the eager result bit for bit (the kernels are deterministic) and the CPU
oracle's result within the tolerance of its dtype.
"""
import numpy as np
import pytest
import torch

from mamba_ssd_scan_chunk_amd import binding as bd
from mamba_ssd_scan_chunk_amd import synth
from tests.gpu_utils import TOL_BF16, TOL_STATE, announce, f64, rel_err

pytestmark = pytest.mark.gpu


def _decode_setup(B=2, H=4, P=64, G=1, N=128, K=4, steps=6):
    C = H * P + 2 * G * N
    xbc, dts = synth.make_decode_stream(steps, B, H, P, G, N, "bf16", seed=70)
    w, _ = synth.make_conv(C, K, "bf16", seed=71)
    pre = synth.make_prefill(B, 1, H, P, G, N, "bf16", seed=72)
    state0 = synth.make_state(B, H, P, N, seed=73, scale=0.3).cuda()
    conv0 = synth.make_tokens(B, K - 1, C, "bf16", seed=74).transpose(1, 2).contiguous().cuda()
    return dict(B=B, H=H, P=P, G=G, N=N, K=K, C=C, steps=steps, xbc=xbc.cuda(), dts=dts.cuda(), w=w.cuda(),
                A_log=pre["A_log"].cuda(), D=pre["D"].cuda(), state0=state0, conv0=conv0)


def _run_steps(s, state, conv, ys):
    H, P, G, N, C = s["H"], s["P"], s["G"], s["N"], s["C"]
    for i in range(s["steps"]):
        row = s["xbc"][i]
        bd.ssd_decode_step(row[:, :H * P], s["dts"][i], s["A_log"], row[:, H * P:H * P + G * N],
                           row[:, H * P + G * N:], s["D"], state, y_t=ys[i], in_stride=C, G=G,
                           conv_state_in=conv[i & 1], conv_state_out=conv[(i + 1) & 1], conv_w=s["w"], K=s["K"],
                           activation=1)


def _decode_oracle(oracle, s):
    """The oracle's run of the same steps: outputs [steps, B, H, P], the
    final state and the final conv window."""
    H, P, G, N, C = s["H"], s["P"], s["G"], s["N"], s["C"]
    xbc, dts = s["xbc"].cpu(), s["dts"].cpu()
    st, cv = f64(s["state0"]), f64(s["conv0"])
    ys = []
    for i in range(s["steps"]):
        r = xbc[i]
        y, st, cv = oracle.decode_step(r[:, :H * P], dts[i], s["A_log"].cpu(), r[:, H * P:H * P + G * N],
                                       r[:, H * P + G * N:], s["D"].cpu(), st, conv_state=cv,
                                       conv_w=s["w"].cpu(), activation=True)
        ys.append(y)
    return np.stack(ys), st, cv


def test_decode_loop_graph_replays_match_eager(oracle):
    s = _decode_setup()
    announce("graph decode")
    ys_o, st_o, cv_o = _decode_oracle(oracle, s)
    ys_ref = torch.empty((s["steps"], s["B"], s["H"], s["P"]), dtype=torch.bfloat16, device="cuda")
    st_ref = s["state0"].clone()
    cv_ref = [s["conv0"].clone(), torch.empty_like(s["conv0"])]
    _run_steps(s, st_ref, cv_ref, ys_ref)
    torch.cuda.synchronize()

    state = s["state0"].clone()
    conv = [s["conv0"].clone(), torch.empty_like(s["conv0"])]
    ys = torch.empty_like(ys_ref)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run_steps(s, state, conv, ys)  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _run_steps(s, state, conv, ys)
    other = s["state0"].clone()
    for rep in range(3):
        # restore the cache eagerly, do unrelated eager work, then replay
        state.copy_(s["state0"])
        conv[0].copy_(s["conv0"])
        ys.zero_()
        _run_steps(s, other, [s["conv0"].clone(), torch.empty_like(s["conv0"])],
                   torch.empty_like(ys_ref))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys, ys_ref), rep
        assert torch.equal(state, st_ref), rep
        final = conv[s["steps"] & 1]
        assert torch.equal(final, cv_ref[s["steps"] & 1]), rep
        assert rel_err(ys, ys_o) <= TOL_BF16, rep
        assert rel_err(state, st_o) <= TOL_STATE, rep
        np.testing.assert_array_equal(f64(final), cv_o)


def test_prefill_graph_replays_match_eager(oracle):
    w = synth.WORKLOADS["mamba2-130m-prefill"]
    dc = synth.make_prefill(w.B, 1000, w.H, w.P, w.G, w.N, w.dtype, seed=75)
    d = {k: v.cuda() for k, v in dc.items()}
    announce("graph prefill")
    y_o, fs_o = oracle.ssd_scan(dc["x"], dc["dt"], dc["A_log"], dc["Bm"], dc["Cm"], dc["D"])
    y_ref, fs_ref = bd.ssd_prefill(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], Q=w.Q)
    torch.cuda.synchronize()
    y = torch.empty_like(y_ref)
    fs = torch.empty_like(fs_ref)
    need = bd.ssd_prefill_workspace_bytes(w.B, 1000, w.H, w.P, w.G, w.N, w.Q, bd.SSD_BF16)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")

    def call():
        bd.ssd_prefill(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], Q=w.Q, y=y, final_state=fs,
                       workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        y.zero_()
        fs.zero_()
        ws.fill_(0xAB)
        bd.ssd_prefill(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], None, Q=w.Q)  # unrelated eager call
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), rep
        assert torch.equal(fs, fs_ref), rep
        assert rel_err(y, y_o) <= TOL_BF16, rep
        assert rel_err(fs, fs_o) <= TOL_BF16, rep


def _capture(call):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()  # warm-up outside capture
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    return g


@pytest.mark.parametrize("H,lengths", [(4, [300, 0, 1, 513, 40]), (64, [300, 0, 1, 513, 40, 700, 260])],
                         ids=["four-kernel-h4", "chained-h64"])
def test_packed_serving_graph_replays_match_eager(oracle, H, lengths):
    """conv over packed prompts, the packed prefill (its chunk tables built on
    the device inside the graph) and the gated normalisation of its output,
    captured as one graph: every replay equals the eager result, and the
    oracle's conv, scan and normalisation (the last on the GPU's y, its
    exact input).  At H = 64 the prefill launches both forms and the chunk
    table picks the chained pass (64 * 12 chunks / 3 >= 192)."""
    P, G, N, K = 64, 1, 128, 4
    T, C = sum(lengths), H * P + 2 * G * N
    dc = synth.make_varlen(lengths, H, P, G, N, "bf16", seed=76)
    d = {k: v.cuda() for k, v in dc.items()}
    xbc_c = synth.make_tokens(1, T, C, "bf16", seed=77)[0]
    xbc = xbc_c.cuda()
    cw_c, cb_c = synth.make_conv(C, K, "bf16", seed=78, with_bias=True)
    cw, cb = cw_c.cuda(), cb_c.cuda()
    z_c, nw_c = synth.make_gate((T,), H * P, "bf16", seed=79)
    z, nw = z_c.cuda(), nw_c.cuda()
    cst0_c = synth.make_tokens(len(lengths), K - 1, C, "bf16", seed=80).transpose(1, 2).contiguous()
    cst0 = cst0_c.cuda()
    cst_o, xc_o = oracle.conv_update_varlen(cst0_c, xbc_c, dc["cu_seqlens"], cw_c, cb_c, True)
    y_o, fs_o = oracle.ssd_scan_varlen(dc["x"], dc["dt"], dc["A_log"], dc["Bm"], dc["Cm"], dc["cu_seqlens"],
                                       dc["D"])
    cu = d["cu_seqlens"]
    B = len(lengths)
    cws = torch.empty(bd.lib().conv_state_update_varlen_workspace_bytes(B, T), dtype=torch.uint8, device="cuda")
    pws = torch.empty(bd.lib().ssd_prefill_varlen_workspace_bytes(B, T, H, P, G, N, 256, bd.SSD_BF16),
                      dtype=torch.uint8, device="cuda")
    cst, xc = cst0.clone(), torch.empty_like(xbc)
    y = torch.empty((T, H, P), dtype=torch.bfloat16, device="cuda")
    fs = torch.empty((B, H, P, N), dtype=torch.float32, device="cuda")
    out = torch.empty((T, H * P), dtype=torch.bfloat16, device="cuda")

    def call():
        bd.conv_state_update_varlen(cst, xbc, cu, cw, cb, activation=1, out=xc, workspace=cws)
        bd.ssd_prefill_varlen(d["x"], d["dt"], d["A_log"], d["Bm"], d["Cm"], d["D"], cu, Q=256, y=y,
                              final_state=fs, workspace=pws)
        bd.ssd_gated_rmsnorm(y.reshape(T, H * P), z, nw, group=H * P, out=out)

    announce("graph packed serving", H)
    call()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (cst, xc, y, fs, out)]
    g = _capture(call)
    for rep in range(3):
        cst.copy_(cst0)
        for t in (xc, y, fs, out):
            t.zero_()
        cws.fill_(0xCD)
        pws.fill_(0xAB)
        # unrelated eager work on the same library between replays
        bd.ssd_gated_rmsnorm(torch.ones((3, 512), dtype=torch.bfloat16, device="cuda"), group=512)
        torch.cuda.synchronize()
        cst.copy_(cst0)
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((cst, xc, y, fs, out), ref):
            assert torch.equal(got, want), rep
        np.testing.assert_array_equal(f64(cst), cst_o)
        assert rel_err(xc, xc_o) <= 8e-3, rep
        assert rel_err(y, y_o) <= TOL_BF16, rep
        assert rel_err(fs, fs_o) <= TOL_BF16, rep
        out_o = oracle.gated_rmsnorm(y.reshape(T, H * P).cpu(), z_c, nw_c, group=H * P)
        assert rel_err(out, out_o) <= 8e-3, rep
