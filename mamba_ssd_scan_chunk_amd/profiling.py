"""Turn rocprofv3 output into the text summaries kept under profiles/.

    python -m mamba_ssd_scan_chunk_amd.profiling stats DIR --command "..." > profiles/<name>.md
        per-kernel table from a `rocprofv3 --kernel-trace --stats --output-format csv` run

    python -m mamba_ssd_scan_chunk_amd.profiling traffic --kernel NAME --fetch DIR --write DIR \
            --command-fetch "..." --command-write "..." --out profiles/traffic_NAME.json
        HBM bytes per launch of NAME from two `rocprofv3 --pmc` runs (FETCH_SIZE,
        then WRITE_SIZE) of a command that also runs bench.py's copy leg: the
        counters of that plain 256 MiB read + 256 MiB write (torch.neg)
        calibrate both counters to bytes.

    python -m mamba_ssd_scan_chunk_amd.profiling mfma --pmc DIR --stats DIR --kernels K1 K2 ... \
            --command-pmc "..." --command-stats "..." --out profiles/mfma_NAME.json > profiles/mfma_NAME.md
        MFMA work and utilisation per kernel from a `rocprofv3 --pmc
        SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES ...` run and a
        kernel-trace run of the same command, which also runs bench.py's gemm
        leg: that bf16 GEMM of known flops checks the counter's unit (512 flops
        per MOP) and shows what a library GEMM reaches by the same measure.

bench.py reads the traffic and MFMA files and reports their figures only
while the kernel sources still hash to the recorded value.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import re
import json
import os
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
COPY_BYTES = 4 * 64 * 2**20  # bench.py copy leg: bytes read and bytes written per dispatch


def _code_only(text: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed, so
    that an edit of comments alone keeps a measurement valid.  String and
    character literals are kept as they are."""
    out, i, n = [], 0, len(text)
    while i < n:
        ch = text[i]
        if ch in "\"'":
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(ch)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def source_hash(files) -> str:
    """Hash of the code (not the comments) of `files`, relative to the
    repository root."""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _find(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def _short(name: str) -> str:
    """Bare kernel name: no namespaces, template arguments or parameters."""
    base = name.replace("(anonymous namespace)", "").strip().strip('"')
    if base.startswith("void "):
        base = base[5:]
    depth, cut = 0, len(base)
    for i, ch in enumerate(base):  # first '(' or '<' at template depth 0
        if ch == "<":
            if depth == 0:
                cut = min(cut, i)
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            cut = min(cut, i)
            break
    return base[:cut].split("::")[-1]


def counter_means(d: str, counter: str) -> dict:
    """Mean over dispatches of a counter (summed over its dimensions), per kernel."""
    per = defaultdict(float)
    kname = {}
    with open(_find(d, "counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            per[r["Dispatch_Id"]] += float(r["Counter_Value"])
            kname[r["Dispatch_Id"]] = r["Kernel_Name"]
    acc = defaultdict(list)
    for disp, v in per.items():
        acc[kname[disp]].append(v)
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def _pick(means: dict, pattern: str, exact: bool):
    hits = [k for k in means if (_short(k) == pattern if exact else pattern in k)]
    return hits[0] if len(hits) == 1 else None


def cmd_traffic(a) -> int:
    fetch = counter_means(a.fetch, "FETCH_SIZE")
    write = counter_means(a.write, "WRITE_SIZE")
    ckf, ckw = _pick(fetch, a.copy_kernel, False), _pick(write, a.copy_kernel, False)
    kf, kw = _pick(fetch, a.kernel, True), _pick(write, a.kernel, True)
    if not (ckf and ckw and kf and kw):
        print(f"kernels seen: {sorted(_short(k) for k in fetch)}", file=sys.stderr)
        return 1
    f_fetch = COPY_BYTES / (fetch[ckf][0] * 1024.0)
    f_write = COPY_BYTES / (write[ckw][0] * 1024.0)
    fb = fetch[kf][0] * 1024.0 * f_fetch
    wb = write[kw][0] * 1024.0 * f_write
    ck = _short(ckf)
    sources = a.sources or []
    rec = {
        "kernel": a.kernel,
        "bytes_per_launch": round(fb + wb),
        "fetch_bytes": round(fb),
        "write_bytes": round(wb),
        "counters_kib_per_dispatch": {"FETCH_SIZE": fetch[kf][0], "WRITE_SIZE": write[kw][0],
                                      "dispatches": fetch[kf][1]},
        "calibration": {"copy_kernel": ck, "copy_bytes_each_way": COPY_BYTES,
                        "copy_FETCH_SIZE_kib": fetch[ckf][0], "copy_WRITE_SIZE_kib": write[ckw][0],
                        "fetch_factor": f_fetch, "write_factor": f_write},
        "commands": {"fetch": a.command_fetch, "write": a.command_write},
        "sources": sources,
        "source_hash": source_hash(sources),
    }
    with open(a.out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(json.dumps(rec))
    return 0


CLOCK_HZ = 2.4e9        # MI355X peak engine clock
SIMDS = 256 * 4         # compute units x SIMDs per CU
MOP_FLOPS = 512         # flops per unit of SQ_INSTS_VALU_MFMA_MOPS_*


def kernel_durations_ns(d: str) -> dict:
    """Average duration (ns) and call count per bare kernel name from a
    `--kernel-trace --stats` run."""
    out = {}
    for r in csv.DictReader(open(_find(d, "kernel_stats.csv"))):
        out[r["Name"]] = (float(r["AverageNs"]), int(r["Calls"]))
    return out


def cmd_mfma(a) -> int:
    mops = counter_means(a.pmc, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    busy = counter_means(a.pmc, "SQ_VALU_MFMA_BUSY_CYCLES")
    durs = kernel_durations_ns(a.stats)
    peak = CLOCK_HZ * SIMDS * 1024  # flops/s: a 32x32x16 bf16 MFMA is 32768 flops in 32 cycles of one SIMD

    def entry(pattern, exact):
        km, kb, kd = _pick(mops, pattern, exact), _pick(busy, pattern, exact), _pick(durs, pattern, exact)
        if not (km and kb and kd):
            raise KeyError(f"{pattern}: seen {sorted(_short(k) for k in mops)}")
        flops = mops[km][0] * MOP_FLOPS
        dur = durs[kd][0] * 1e-9
        return {"mops_bf16": mops[km][0], "flops": flops, "mfma_busy_cycles": busy[kb][0],
                "avg_us": round(dur * 1e6, 3), "calls_traced": durs[kd][1], "dispatches_counted": mops[km][1],
                "tflops": round(flops / dur / 1e12, 2),
                "busy_frac": round(busy[kb][0] / (dur * CLOCK_HZ * SIMDS), 4),
                "peak_frac": round(flops / dur / peak, 4)}

    kernels = {k: entry(k, True) for k in a.kernels}
    gemm = entry(a.gemm_kernel, False)
    gemm["flops_expected"] = a.gemm_flops
    sources = a.sources or []
    rec = {"workload": a.workload, "kernels": kernels, "gemm_reference": gemm, "peak_tflops": peak / 1e12,
           "clock_hz": CLOCK_HZ, "simds": SIMDS,
           "commands": {"pmc": a.command_pmc, "stats": a.command_stats},
           "sources": sources, "source_hash": source_hash(sources)}
    with open(a.out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    print(f"# rocprofv3 MFMA counters: {a.title}\n")
    print("Commands (from the repository root on an MI355X):\n")
    print(f"```\n{a.command_pmc}\n{a.command_stats}\n```\n")
    print("Executed MFMA flops = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 per dispatch; the MFMA busy fraction is "
          f"SQ_VALU_MFMA_BUSY_CYCLES / (average kernel-trace duration x {CLOCK_HZ / 1e9:g} GHz x {SIMDS} SIMDs); "
          f"the peak is {peak / 1e12:.0f} TFLOP/s (listed by AMD as 2.5 PFLOP/s).\n")
    print("| Kernel | MOPS_BF16 per dispatch | Executed GFLOP | MFMA busy cycles (sum over SIMDs) | "
          "Average duration (us) | TFLOP/s | MFMA busy | Share of the bf16 peak |")
    print("|---|---|---|---|---|---|---|---|")
    for name, e in list(kernels.items()) + [(f"{a.gemm_kernel}... (torch.matmul, reference)", gemm)]:
        print(f"| {name} | {e['mops_bf16']:.0f} | {e['flops'] / 1e9:.3f} | {e['mfma_busy_cycles']:.0f} | "
              f"{e['avg_us']:.2f} | {e['tflops']:.1f} | {100 * e['busy_frac']:.1f}% | {100 * e['peak_frac']:.1f}% |")
    tot_f = sum(e["flops"] for e in kernels.values())
    tot_t = sum(e["avg_us"] for e in kernels.values()) * 1e-6
    print(f"\nAll listed kernels together: {tot_f / 1e9:.3f} GFLOP executed in {tot_t * 1e6:.1f} us of kernel time, "
          f"{tot_f / tot_t / 1e12:.1f} TFLOP/s = {100 * tot_f / tot_t / peak:.1f}% of the peak.")
    print(f"\nGEMM reference: counted {gemm['flops']:.6g} flops against 2 x {a.gemm_n}^3 = {a.gemm_flops:.6g} "
          f"(ratio {gemm['flops'] / a.gemm_flops:.6f}).")
    return 0


def cmd_stats(a) -> int:
    rows = list(csv.DictReader(open(_find(a.dir, "kernel_stats.csv"))))
    print(f"# rocprofv3 kernel statistics: {a.title}\n")
    print(f"Command (from the repository root on an MI355X):\n\n```\n{a.command}\n```\n")
    print("| Kernel | Calls | Average (us) | Min (us) | Max (us) | Share of GPU time |")
    print("|---|---|---|---|---|---|")
    for r in rows:
        name = _short(r["Name"])
        print(f"| {name} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
              f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--kernel", required=True)
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-kernel", default="neg_kernel",
                   help="substring naming bench.py's copy-leg kernel (torch.neg over 256 MiB)")
    t.add_argument("--command-fetch", default="")
    t.add_argument("--command-write", default="")
    t.add_argument("--sources", nargs="*")
    t.add_argument("--out", required=True)
    st = sub.add_parser("stats")
    st.add_argument("dir")
    st.add_argument("--title", default="")
    st.add_argument("--command", default="")
    m = sub.add_parser("mfma")
    m.add_argument("--pmc", required=True)
    m.add_argument("--stats", required=True)
    m.add_argument("--kernels", nargs="+", required=True)
    m.add_argument("--gemm-kernel", default="Cijk_", help="substring naming the gemm leg's library kernel")
    m.add_argument("--gemm-n", type=int, default=8192)
    m.add_argument("--workload", required=True, help="bench.py workload name the counters were taken on")
    m.add_argument("--title", default="")
    m.add_argument("--command-pmc", default="")
    m.add_argument("--command-stats", default="")
    m.add_argument("--sources", nargs="*")
    m.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "mfma":
        a.gemm_flops = 2 * a.gemm_n ** 3
        return cmd_mfma(a)
    return cmd_traffic(a) if a.cmd == "traffic" else cmd_stats(a)


if __name__ == "__main__":
    sys.exit(main())
