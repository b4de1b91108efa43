"""Turn rocprofv3 output into the text summaries kept under profiles/.

    python -m mamba_ssd_scan_chunk_amd.profiling stats DIR --command "..." > profiles/<name>.md
        per-kernel table from a `rocprofv3 --kernel-trace --stats --output-format csv` run

    python -m mamba_ssd_scan_chunk_amd.profiling traffic --kernel NAME --fetch DIR --write DIR \
            --command-fetch "..." --command-write "..." --out profiles/traffic_NAME.json
        HBM bytes per launch of NAME from two `rocprofv3 --pmc` runs (FETCH_SIZE,
        then WRITE_SIZE) of a command that also runs bench.py's copy leg: the
        counters of that plain 256 MiB read + 256 MiB write (torch.neg)
        calibrate both counters to bytes.

bench.py reads the traffic files and reports their bytes only while the
kernel sources still hash to the recorded value.
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
    a = ap.parse_args(argv)
    return cmd_traffic(a) if a.cmd == "traffic" else cmd_stats(a)


if __name__ == "__main__":
    sys.exit(main())
