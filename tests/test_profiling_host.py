"""Host logic of the rocprofv3 summaries (mamba_ssd_scan_chunk_amd.profiling)
on small hand-made CSV files: the counter-to-bytes calibration, the MFMA
flop and busy-fraction arithmetic, kernel-name matching and the source hash
that keeps a measurement tied to the code it was taken on."""
import csv
import json
import os

import pytest

from mamba_ssd_scan_chunk_amd import profiling as prof

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def _write_stats(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_kernel_stats.csv"), "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"])
        for name, calls, avg in rows:
            w.writerow([name, calls, calls * avg, avg, 50.0, avg, avg, 0.0])


K_OUT = "ssd::(anonymous namespace)::chunk_out_mfma(ssd::PrefillArgs)"
K_GEMM = "Cijk_Ailk_Bljk_BBS_BH_MT256x256x64"


def test_short_names():
    assert prof._short(K_OUT) == "chunk_out_mfma"
    assert prof._short("void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel>(int)") == \
        "vectorized_elementwise_kernel"
    assert prof._short("ssd::(anonymous namespace)::decode_step_kernel<float, 128, true, 4, 4>(ssd::DecodeArgs)") == \
        "decode_step_kernel"


def test_counter_means_sum_dimensions_then_average_dispatches(tmp_path):
    d = str(tmp_path / "p")
    _write_counters(d, [(1, K_OUT, "FETCH_SIZE", 10), (1, K_OUT, "FETCH_SIZE", 6),
                        (2, K_OUT, "FETCH_SIZE", 20), (3, K_OUT, "WRITE_SIZE", 99)])
    assert prof.counter_means(d, "FETCH_SIZE") == {K_OUT: (18.0, 2)}


def test_traffic_calibration(tmp_path):
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"
    # the copy reads and writes COPY_BYTES; FETCH counts half of what it reads
    cb = prof.COPY_BYTES / 1024.0
    f, w = str(tmp_path / "f"), str(tmp_path / "w")
    _write_counters(f, [(1, copy, "FETCH_SIZE", cb / 2), (2, K_OUT, "FETCH_SIZE", 1000.0)])
    _write_counters(w, [(1, copy, "WRITE_SIZE", cb), (2, K_OUT, "WRITE_SIZE", 500.0)])
    out = str(tmp_path / "t.json")
    assert prof.main(["traffic", "--kernel", "chunk_out_mfma", "--fetch", f, "--write", w,
                      "--copy-kernel", "neg_kernel", "--out", out]) == 0
    rec = json.load(open(out))
    assert rec["fetch_bytes"] == 2 * 1000 * 1024
    assert rec["write_bytes"] == 500 * 1024
    assert rec["bytes_per_launch"] == 2500 * 1024


def test_mfma_flops_and_busy_fraction(tmp_path, capsys):
    p, s = str(tmp_path / "p"), str(tmp_path / "s")
    n = 64
    gemm_mops = 2 * n ** 3 / 512
    _write_counters(p, [(1, K_OUT, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e6), (1, K_OUT, "SQ_VALU_MFMA_BUSY_CYCLES", 5e5),
                        (2, K_GEMM, "SQ_INSTS_VALU_MFMA_MOPS_BF16", gemm_mops),
                        (2, K_GEMM, "SQ_VALU_MFMA_BUSY_CYCLES", gemm_mops / 2)])
    _write_stats(s, [(K_OUT, 10, 2000.0), (K_GEMM, 3, 1000.0)])
    out = str(tmp_path / "m.json")
    assert prof.main(["mfma", "--workload", "w", "--pmc", p, "--stats", s, "--kernels", "chunk_out_mfma",
                      "--gemm-n", str(n), "--out", out]) == 0
    rec = json.load(open(out))
    k = rec["kernels"]["chunk_out_mfma"]
    assert k["flops"] == 512 * 1e6
    assert k["tflops"] == pytest.approx(512e6 / 2e-6 / 1e12, rel=1e-3)
    # busy cycles / (duration x clock x SIMDs); flops / (duration x peak) agree when busy = MOPS / 2
    assert k["busy_frac"] == pytest.approx(5e5 / (2e-6 * prof.CLOCK_HZ * prof.SIMDS), rel=1e-2)
    assert k["peak_frac"] == pytest.approx(k["busy_frac"], rel=1e-2)
    assert rec["gemm_reference"]["flops"] == 2 * n ** 3
    assert rec["workload"] == "w"
    assert "ratio 1.000000" in capsys.readouterr().out


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    monkeypatch.setattr(prof, "ROOT", str(tmp_path))
    src = tmp_path / "k.hip"
    src.write_text("int f(int a) { return a + 1; } // one\n/* two */\n")
    h0 = prof.source_hash(["k.hip"])
    src.write_text("// changed comment\nint f(int a) {\n  return a + 1;\n}\n")
    assert prof.source_hash(["k.hip"]) == h0
    src.write_text("int f(int a) { return a + 2; }\n")
    assert prof.source_hash(["k.hip"]) != h0
    src.write_text('const char *s = "// not a comment"; int f(int a) { return a + 1; }\n')
    assert prof.source_hash(["k.hip"]) != h0


def test_committed_summaries_are_current():
    """The committed traffic and MFMA files were taken on the kernel sources
    as they are (bench.py reports them only then)."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    names = [f for f in os.listdir(os.path.join(root, "profiles")) if f.endswith(".json")]
    assert names
    for f in names:
        rec = json.load(open(os.path.join(root, "profiles", f)))
        assert rec["source_hash"] == prof.source_hash(rec["sources"]), f
