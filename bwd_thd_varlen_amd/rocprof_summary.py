"""Text summaries of rocprofv3 result databases for ``profiles/``.

Two modes, each run on the databases a GPU run left behind:

  python -m bwd_thd_varlen_amd.rocprof_summary trace DB OUT.md --command CMD [--title T]
      kernel-trace summary (calls, average and total duration per kernel)
      from the ``top_kernels`` view of a ``rocprofv3 --kernel-trace --stats``
      database.

  python -m bwd_thd_varlen_amd.rocprof_summary traffic FETCH_DB WRITE_DB \\
          --command-fetch CMD --command-write CMD
      HBM traffic per launch of each compute kernel from two counter runs
      (``--pmc FETCH_SIZE`` and ``--pmc WRITE_SIZE``) of ``bench.py
      --copy-calibration``.  The counters (KiB per dispatch) are scaled by
      what they read for the plain 1 GiB device copies that option adds, so
      that a copy of N bytes counts N bytes read and N written.  Writes
      ``profiles/<stage>_throughput_65k_pmc.txt`` for fwd, dq and dkdv,
      stamped with the hash of the kernel sources (``source_hash``);
      bench.py reports the traffic only while that hash matches.

  python -m bwd_thd_varlen_amd.rocprof_summary counters OUT.txt DB [DB ...] --command CMD [...]
          [--workload throughput_65k|d256_65k]
      shader-sequencer counters of the three compute kernels from one or more
      ``rocprofv3 --pmc`` runs (at most 8 SQ counters per run), averaged per
      dispatch, with the wave-cycle ratios they give.  ``--workload d256_65k``
      picks the head-dim-256 kernels (the split dQ and dK/dV kernels) instead
      of the d=128 ones.

Reads SQLite files only; nothing here touches the GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import os
import re
import sqlite3
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")

# kernel sources behind each timed stage (a change to any of them makes a
# stored counter summary stale)
KERNEL_SOURCES = {
    "fwd": ["bwd_thd_varlen_amd/csrc/fwd.hip", "bwd_thd_varlen_amd/csrc/common.h"],
    "dq": ["bwd_thd_varlen_amd/csrc/bwd.hip", "bwd_thd_varlen_amd/csrc/common.h"],
    "dkdv": ["bwd_thd_varlen_amd/csrc/bwd.hip", "bwd_thd_varlen_amd/csrc/common.h"],
}

# demangled-name prefixes of each stage's kernel for the bf16 d=128 causal workload
STAGE_KERNELS = {
    "fwd": "void attn::fwd_kernel<0, 128, true",
    "dq": "void attn::dq_kernel<0, 128, true",
    "dkdv": "void attn::dkdv_kernel<0, 128, true",
}
# the same for the head-dim-256 workload (split dQ and dK/dV kernels)
STAGE_KERNELS_D256 = {
    "fwd": "void attn::fwd_kernel<0, 256, true",
    "dq": "void attn::dq_split_kernel<0, true",
    "dkdv": "void attn::dkdv_split_kernel<0, true",
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"
COPY_BYTES = 1 << 30          # bench.py --copy-calibration: 1 GiB copies
COPY_MIN_KIB = (COPY_BYTES >> 10) // 4   # smaller copies (argument uploads) are ignored


def code_only(text: str) -> str:
    """A C++ source without its comments, trailing blanks and blank lines, so
    that an edit to a comment leaves the hash below (and with it every stored
    summary) as it is."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_hash(stage: str) -> str:
    """sha256 (16 hex digits) of the code of the stage's kernel sources."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES.get(stage, []):
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


def _rows(db: str, sql: str):
    con = sqlite3.connect(db)
    try:
        return list(con.execute(sql))
    finally:
        con.close()


TRACE_TITLE = "throughput_65k (65536 tokens, hq=64 hkv=8 d=128, bf16, padding_causal)"


def trace(db: str, out: str, command: str, title: str = TRACE_TITLE) -> None:
    rows = _rows(db, "select * from top_kernels")
    total = sum(r[2] for r in rows)
    lines = [
        f"# Kernel trace: {title}",
        "",
        "Command (run from the repository root on one MI355X, `TMPDIR=/tmp`):",
        "",
        f"    {command}",
        "",
        "Durations in microseconds, from the `top_kernels` view of the rocprofv3",
        "results database (every dispatch of the run: warm-up and timed steps);",
        "median and minimum from the per-dispatch `kernels` view.",
        "",
        "| kernel | calls | avg us | median us | min us | total us | share |",
        "|---|---|---|---|---|---|---|",
    ]
    per = defaultdict(list)
    for name, dur in _rows(db, "select name, end - start from kernels"):
        per[name].append(dur / 1000.0)
    for name, calls, tot, avg, *_ in rows:
        short = name.split("(")[0].replace("void ", "")
        ds = sorted(per.get(name, [avg]))
        med = 0.5 * (ds[(len(ds) - 1) // 2] + ds[len(ds) // 2])
        lines.append(f"| {short} | {calls} | {avg:.1f} | {med:.1f} | {ds[0]:.1f} | {tot:.1f} "
                     f"| {100.0 * tot / total:.2f}% |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def _counter(db: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter."""
    out = defaultdict(list)
    for name, value in _rows(db, "select kernel_name, value from counters_collection "
                                 f"where counter_name = '{counter}' order by dispatch_id"):
        out[name].append(float(value))
    return out


def _copy_scale(values: dict) -> tuple:
    big = [v for name, vs in values.items() if name.startswith(COPY_KERNEL) for v in vs
           if v >= COPY_MIN_KIB]
    if not big:
        raise SystemExit("no 1 GiB copy dispatch found: run bench.py with --copy-calibration")
    mean = sum(big) / len(big)
    return (COPY_BYTES / 1024.0) / mean, len(big), mean


def traffic(fetch_db: str, write_db: str, cmd_fetch: str, cmd_write: str) -> None:
    fetch, write = _counter(fetch_db, "FETCH_SIZE"), _counter(write_db, "WRITE_SIZE")
    fscale, fn, fmean = _copy_scale(fetch)
    wscale, wn, wmean = _copy_scale(write)
    for stage, prefix in STAGE_KERNELS.items():
        fv = [v for name, vs in fetch.items() if name.startswith(prefix) for v in vs]
        wv = [v for name, vs in write.items() if name.startswith(prefix) for v in vs]
        if not fv or not wv:
            print(f"{stage}: kernel {prefix!r} not in both databases, skipped")
            continue
        kname = next(name for name in fetch if name.startswith(prefix))
        f_kib, w_kib = sum(fv) / len(fv), sum(wv) / len(wv)
        hbm = (f_kib * fscale + w_kib * wscale) * 1024.0
        path = os.path.join(PROFILES, f"{stage}_throughput_65k_pmc.txt")
        with open(path, "w") as f:
            f.write(
                f"# HBM traffic per launch: {kname.split('(')[0]}, throughput_65k workload\n"
                "# Two counter runs, from the repository root on one MI355X (TMPDIR=/tmp):\n"
                f"#   {cmd_fetch}\n"
                f"#   {cmd_write}\n"
                "# FETCH_SIZE / WRITE_SIZE are KiB per dispatch; each is scaled by\n"
                "# 1 GiB / (its value for the 1 GiB device copies of --copy-calibration).\n"
                f"kernel_source_sha256 = {source_hash(stage)}\n"
                f"dispatches = {len(fv)}\n"
                f"fetch_kib_per_launch = {f_kib:.1f}\n"
                f"write_kib_per_launch = {w_kib:.1f}\n"
                f"copy_fetch_kib = {fmean:.1f}\n"
                f"copy_write_kib = {wmean:.1f}\n"
                f"copy_dispatches = {min(fn, wn)}\n"
                f"fetch_scale = {fscale:.4f}\n"
                f"write_scale = {wscale:.4f}\n"
                f"hbm_bytes_per_launch = {hbm:.0f}\n")
        print(f"wrote {path}: {hbm / 2**30:.3f} GiB per launch")


# ratios of wave-cycle counters (each summed over all waves of a dispatch)
RATIOS = [
    ("waiting on anything", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
    ("waiting on an instruction's dependency", "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
    ("waiting on LDS", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"),
    ("issuing any instruction", "SQ_ACTIVE_INST_ANY", "SQ_WAVE_CYCLES"),
    ("issuing VALU (MFMA included)", "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES"),
    ("issuing LDS", "SQ_ACTIVE_INST_LDS", "SQ_WAVE_CYCLES"),
    ("issuing scalar", "SQ_ACTIVE_INST_SCA", "SQ_WAVE_CYCLES"),
]
# per LDS instruction: bank-conflict cycles (0 = conflict-free)
LDS_RATIOS = [
    ("bank-conflict cycles per LDS instruction", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS"),
    ("bank-conflict cycles per LDS-busy cycle", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS"),
]
XCDS = 8   # GRBM counters are summed over the accelerator's 8 XCDs


def counters(out: str, dbs, commands, workload: str = "throughput_65k") -> None:
    kernels = STAGE_KERNELS_D256 if workload == "d256_65k" else STAGE_KERNELS
    vals = defaultdict(lambda: defaultdict(list))
    durs = defaultdict(list)
    for db in dbs:
        for name, counter, value, dur in _rows(db, "select kernel_name, counter_name, value, "
                                                   "duration from counters_collection"):
            for stage, prefix in kernels.items():
                if name.startswith(prefix):
                    vals[stage][counter].append(float(value))
                    durs[stage].append(float(dur))
    names = sorted({c for st in vals.values() for c in st})
    lines = [f"# Shader-sequencer counters: {workload} workload, per dispatch (average)",
             "# kernels: " + ", ".join(f"{st} = {pre.split('attn::')[1]}..." for st, pre in kernels.items()),
             "# Counter runs, from the repository root on one MI355X (TMPDIR=/tmp):"]
    lines += [f"#   {c}" for c in commands]
    for stage in STAGE_KERNELS:
        lines.append(f"kernel_source_sha256[{stage}] = {source_hash(stage)}")
    lines += ["", "| counter | " + " | ".join(STAGE_KERNELS) + " |",
              "|---|" + "---|" * len(STAGE_KERNELS)]
    avg = {st: {c: sum(v) / len(v) for c, v in d.items()} for st, d in vals.items()}
    for c in names:
        lines.append(f"| {c} | " + " | ".join(f"{avg.get(st, {}).get(c, float('nan')):.4g}"
                                              for st in STAGE_KERNELS) + " |")
    lines += ["", "| share of wave-cycles | " + " | ".join(STAGE_KERNELS) + " |",
              "|---|" + "---|" * len(STAGE_KERNELS)]
    for label, num, den in RATIOS:
        cells = []
        for st in STAGE_KERNELS:
            a = avg.get(st, {})
            cells.append(f"{100.0 * a[num] / a[den]:.1f}%" if num in a and a.get(den) else "-")
        lines.append(f"| {label} ({num} / {den}) | " + " | ".join(cells) + " |")
    for label, num, den in LDS_RATIOS:
        cells = []
        for st in STAGE_KERNELS:
            a = avg.get(st, {})
            cells.append(f"{a[num] / a[den]:.4g}" if num in a and a.get(den) else "-")
        if any(c != "-" for c in cells):
            lines.append(f"| {label} ({num} / {den}) | " + " | ".join(cells) + " |")
    if any("GRBM_GUI_ACTIVE" in avg.get(st, {}) for st in STAGE_KERNELS):
        cells = []
        for st in STAGE_KERNELS:
            a, d = avg.get(st, {}), durs.get(st)
            ok = "GRBM_GUI_ACTIVE" in a and d
            cells.append(f"{a['GRBM_GUI_ACTIVE'] / XCDS / (sum(d) / len(d)):.2f} GHz" if ok else "-")
        lines.append(f"| shader clock while the kernel runs (GRBM_GUI_ACTIVE / {XCDS} XCDs / "
                     "dispatch duration) | " + " | ".join(cells) + " |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="mode", required=True)
    t = sub.add_parser("trace")
    t.add_argument("db")
    t.add_argument("out")
    t.add_argument("--command", required=True)
    t.add_argument("--title", default=TRACE_TITLE)
    c = sub.add_parser("traffic")
    c.add_argument("fetch_db")
    c.add_argument("write_db")
    c.add_argument("--command-fetch", required=True)
    c.add_argument("--command-write", required=True)
    k = sub.add_parser("counters")
    k.add_argument("out")
    k.add_argument("dbs", nargs="+")
    k.add_argument("--command", action="append", required=True)
    k.add_argument("--workload", default="throughput_65k", choices=["throughput_65k", "d256_65k"])
    a = ap.parse_args(argv)
    if a.mode == "counters":
        counters(a.out, a.dbs, a.command, a.workload)
    elif a.mode == "trace":
        trace(a.db, a.out, a.command, a.title)
    else:
        traffic(a.fetch_db, a.write_db, a.command_fetch, a.command_write)


if __name__ == "__main__":
    main(sys.argv[1:])
