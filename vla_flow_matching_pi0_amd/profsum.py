"""Turn rocprofv3 CSV output into the short text summaries kept with the
library (kernel time statistics, HBM traffic of one kernel).

  python -m vla_flow_matching_pi0_amd.profsum stats <kernel_stats.csv> <out.md> --cmd "<command>" [--match <name part>]
  python -m vla_flow_matching_pi0_amd.profsum traffic <fetch counter_collection.csv> <write counter_collection.csv>
         <out.md> --kernel k_persistent --calib-mib 1024 --cmd-fetch "<command>" --cmd-write "<command>"

The traffic summary scales the FETCH_SIZE / WRITE_SIZE counters (KiB per
dispatch) of the kernel by the ratio of known bytes to counted bytes of a
plain streaming kernel (float32 negation: reads and writes `calib-mib` MiB)
profiled in the same run.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = ["vla_flow_matching_pi0_amd/csrc/vfm_phases.h", "vla_flow_matching_pi0_amd/csrc/vfm_device.h",
                  "vla_flow_matching_pi0_amd/csrc/vfm_params.h", "vla_flow_matching_pi0_amd/csrc/vfm_launch.cpp",
                  "vla_flow_matching_pi0_amd/csrc/vfm_runtime.cpp"]


def source_digest() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def short_name(name: str) -> str:
    name = name.strip()
    if name.startswith("void "):
        name = name[5:]
    return name.split("(")[0][:110]


def stats(path: str, out: str, cmd: str, top: int = 20, match: str = "") -> None:
    rows = [r for r in csv.DictReader(open(path)) if match in r["Name"]]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    title = "# rocprofv3 kernel statistics" + (f" (kernels matching `{match}`)" if match else "")
    lines = [title, "", "Command:", "", "```", cmd, "```", "",
             "| kernel | calls | total ms | average us | min us | max us | % |", "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows[:top]:
        lines.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.3f} | "
                     f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.2f} |")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


def _per_dispatch(path: str, counter: str):
    """{dispatch id: (kernel name, value)} for one counter."""
    acc = collections.defaultdict(float)
    names = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        d = r["Dispatch_Id"]
        acc[d] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    return {d: (names[d], v) for d, v in acc.items()}


def _kernel_and_calib(path: str, counter: str, kernel: str, calib_bytes: int):
    disp = _per_dispatch(path, counter)
    kv = [v for n, v in disp.values() if kernel in n]
    cv = [v for n, v in disp.values() if "neg_kernel" in n and v * 1024 > 0.5 * calib_bytes]
    if not kv or not cv:
        raise SystemExit(f"{path}: no dispatch of {kernel} ({len(kv)}) or of the calibration kernel ({len(cv)})")
    return sum(kv) / len(kv) * 1024, sum(cv) / len(cv) * 1024, len(kv), len(cv)


def traffic(fetch_csv: str, write_csv: str, out: str, kernel: str, calib_mib: int, cmd_fetch: str,
            cmd_write: str, workload: str) -> None:
    cb = calib_mib << 20
    kf, cf, nkf, ncf = _kernel_and_calib(fetch_csv, "FETCH_SIZE", kernel, cb)
    kw, cw, nkw, ncw = _kernel_and_calib(write_csv, "WRITE_SIZE", kernel, cb)
    sf, sw = cb / cf, cb / cw
    fetch, write = kf * sf, kw * sw
    lines = [f"# HBM traffic of `{kernel}` ({workload})", "",
             "FETCH_SIZE and WRITE_SIZE (KiB per dispatch) from two rocprofv3 --pmc runs, each scaled by the "
             f"same counter on a plain float32 negation kernel that reads and writes {calib_mib} MiB.", "",
             "Fetch pass:", "", "```", cmd_fetch, "```", "", "Write pass:", "", "```", cmd_write, "```", "",
             f"- `kernel_dispatches_fetch_pass`: {nkf}",
             f"- `kernel_dispatches_write_pass`: {nkw}",
             f"- `fetch_counter_bytes_per_launch`: {int(kf)}",
             f"- `write_counter_bytes_per_launch`: {int(kw)}",
             f"- `calib_fetch_counter_bytes`: {int(cf)} (known {cb}; scale {sf:.4f})",
             f"- `calib_write_counter_bytes`: {int(cw)} (known {cb}; scale {sw:.4f})",
             f"- `fetch_bytes_per_launch`: {int(fetch)}",
             f"- `write_bytes_per_launch`: {int(write)}",
             f"- `hbm_bytes_per_launch`: {int(fetch + write)}",
             f"- `kernel_source_sha256`: {source_digest()}", ""]
    open(out, "w").write("\n".join(lines))
    print("\n".join(lines))


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="mode", required=True)
    a = sub.add_parser("stats")
    a.add_argument("csv")
    a.add_argument("out")
    a.add_argument("--cmd", required=True)
    a.add_argument("--match", default="", help="keep only kernels whose name contains this")
    b = sub.add_parser("traffic")
    b.add_argument("fetch_csv")
    b.add_argument("write_csv")
    b.add_argument("out")
    b.add_argument("--kernel", default="k_persistent")
    b.add_argument("--workload", default="pi05_bf16_b1")
    b.add_argument("--calib-mib", type=int, required=True)
    b.add_argument("--cmd-fetch", required=True)
    b.add_argument("--cmd-write", required=True)
    args = ap.parse_args(argv)
    if args.mode == "stats":
        stats(args.csv, args.out, args.cmd, match=args.match)
    else:
        traffic(args.fetch_csv, args.write_csv, args.out, args.kernel, args.calib_mib, args.cmd_fetch,
                args.cmd_write, args.workload)
    return 0


if __name__ == "__main__":
    sys.exit(main())
