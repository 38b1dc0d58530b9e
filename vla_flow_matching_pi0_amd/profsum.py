"""Turn rocprofv3 CSV output into the short text summaries kept with the
library (kernel time statistics, HBM traffic of one kernel).

  python -m vla_flow_matching_pi0_amd.profsum stats <kernel_stats.csv> <out.md> --cmd "<command>" [--match <name part>]
  python -m vla_flow_matching_pi0_amd.profsum traffic <fetch counter_collection.csv> <write counter_collection.csv>
         <out.md> --kernel k_persistent --calib-mib 1024 --cmd-fetch "<command>" --cmd-write "<command>"
  python -m vla_flow_matching_pi0_amd.profsum gaps <kernel_trace.csv> <out.md> --match <name part> --cmd "<command>"

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
_C = "vla_flow_matching_pi0_amd/csrc/"
# the sources each timed kernel is built from: a traffic figure taken from
# counters is only reported while it still describes this code
KERNEL_SOURCES = {
    "k_persistent": [_C + "vfm_phases.h", _C + "vfm_device.h", _C + "vfm_params.h", _C + "vfm_launch.cpp",
                     _C + "vfm_runtime.cpp"],
    "k_stream": [_C + "vfm_stream.h", _C + "vfm_stream_params.h", _C + "vfm_k_stream.hip", _C + "vfm_stream_rt.cpp",
                 _C + "vfm_device.h", _C + "vfm_params.h"],
}


def source_digest(kernel: str = "k_persistent") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
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


def _probe_scale(path: str, counter: str, policy: int, calib_bytes: int):
    """known bytes / counted bytes of the copy probe with load policy `policy` (None if absent)."""
    disp = _per_dispatch(path, counter)
    v = [x for n, x in disp.values() if f"k_copy_probe<{policy}>" in n and x * 1024 > 0.5 * calib_bytes]
    return calib_bytes / (sum(v) / len(v) * 1024) if v else None


def traffic(fetch_csv: str, write_csv: str, out: str, kernel: str, calib_mib: int, cmd_fetch: str,
            cmd_write: str, workload: str) -> None:
    cb = calib_mib << 20
    kf, cf, nkf, ncf = _kernel_and_calib(fetch_csv, "FETCH_SIZE", kernel, cb)
    kw, cw, nkw, ncw = _kernel_and_calib(write_csv, "WRITE_SIZE", kernel, cb)
    sf, sw = cb / cf, cb / cw
    probe = {pol: _probe_scale(fetch_csv, "FETCH_SIZE", pol, cb) for pol in (0, 16)}
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
             f"- `fetch_scale_copy_plain_loads`: {probe[0]:.4f}" if probe[0] else "- `fetch_scale_copy_plain_loads`: n/a",
             f"- `fetch_scale_copy_sc1_loads`: {probe[16]:.4f}" if probe[16] else "- `fetch_scale_copy_sc1_loads`: n/a",
             f"- `fetch_bytes_per_launch`: {int(fetch)}",
             f"- `write_bytes_per_launch`: {int(write)}",
             f"- `hbm_bytes_per_launch`: {int(fetch + write)}",
             f"- `kernel_source_sha256`: {source_digest(kernel)}", ""]
    open(out, "w").write("\n".join(lines))
    print("\n".join(lines))


def gaps(path: str, out: str, cmd: str, match: str, skip_frac: float) -> None:
    """Launch-gap share of a kernel-trace timeline: over the dispatches whose
    name contains `match` (the first `skip_frac` of them dropped as warmup),
    the share of the wall span from the first start to the last end during
    which none of them runs."""
    rows = [r for r in csv.DictReader(open(path)) if match in r["Kernel_Name"]]
    iv = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows)
    iv = iv[int(len(iv) * skip_frac):]
    if not iv:
        raise SystemExit(f"{path}: no dispatch matching {match!r}")
    busy, cur_s, cur_e = 0, iv[0][0], iv[0][1]
    for s0, e0 in iv[1:]:
        if s0 > cur_e:
            busy += cur_e - cur_s
            cur_s, cur_e = s0, e0
        else:
            cur_e = max(cur_e, e0)
    busy += cur_e - cur_s
    span = max(e for _, e in iv) - iv[0][0]
    frac = 1.0 - busy / span
    lines = [f"# Launch gaps of the kernels matching `{match}`", "", "Command:", "", "```", cmd, "```", "",
             f"Dispatches after dropping the first {skip_frac:.0%} as warmup: {len(iv)}.", "",
             f"- `span_us`: {span / 1e3:.1f}",
             f"- `busy_us`: {busy / 1e3:.1f}",
             f"- `gap_us`: {(span - busy) / 1e3:.1f}",
             f"- `launch_gap_frac`: {frac:.4f}", ""]
    open(out, "w").write("\n".join(lines))
    print("\n".join(lines))


def mfma(path: str, out: str, cmd: str, match: str = "", top: int = 12) -> None:
    """MFMA activity per kernel from SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE
    (both summed over the device: the busy counter over its 1024 SIMDs, the
    active counter over its 8 XCDs): busy fraction = MFMA busy cycles /
    (1024 x active cycles per XCD), aggregated over each kernel's dispatches."""
    busy = _per_dispatch(path, "SQ_VALU_MFMA_BUSY_CYCLES")
    act = _per_dispatch(path, "GRBM_GUI_ACTIVE")
    agg = collections.defaultdict(lambda: [0, 0.0, 0.0])
    keep = [m for m in match.split(",") if m]
    for d, (name, b) in busy.items():
        if d not in act or (keep and not any(m in name for m in keep)):
            continue
        a = agg[short_name(name)]
        a[0] += 1
        a[1] += b
        a[2] += act[d][1] / 8.0
    rows = sorted(agg.items(), key=lambda kv: -kv[1][2])
    tb = sum(v[1] for v in agg.values())
    ta = sum(v[2] for v in agg.values())
    lines = ["# MFMA activity per kernel", "", "Command:", "", "```", cmd, "```", "",
             "Busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs), summed over "
             "the kernel's dispatches; time share = its active cycles over all kernels counted"
             + (f" (names containing any of: {', '.join(keep)})" if keep else "") + ".", "",
             "| kernel | dispatches | active Mcycles per XCD | time share | MFMA busy |", "|---|---:|---:|---:|---:|"]
    for n, (c, b, a) in rows[:top]:
        lines.append(f"| `{n}` | {c} | {a / 1e6:.2f} | {a / ta:.3f} | {b / (1024 * a):.4f} |")
    lines += ["", f"- `mfma_busy_fraction_counted_kernels`: {tb / (1024 * ta):.4f}", ""]
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
    c = sub.add_parser("gaps")
    c.add_argument("csv")
    c.add_argument("out")
    c.add_argument("--cmd", required=True)
    c.add_argument("--match", required=True)
    c.add_argument("--skip-frac", type=float, default=0.2)
    dm = sub.add_parser("mfma")
    dm.add_argument("csv")
    dm.add_argument("out")
    dm.add_argument("--cmd", required=True)
    dm.add_argument("--match", default="", help="comma-separated name parts; count only kernels matching one")
    args = ap.parse_args(argv)
    if args.mode == "mfma":
        mfma(args.csv, args.out, args.cmd, args.match)
        return 0
    if args.mode == "gaps":
        gaps(args.csv, args.out, args.cmd, args.match, args.skip_frac)
        return 0
    if args.mode == "stats":
        stats(args.csv, args.out, args.cmd, match=args.match)
    else:
        traffic(args.fetch_csv, args.write_csv, args.out, args.kernel, args.calib_mib, args.cmd_fetch,
                args.cmd_write, args.workload)
    return 0


if __name__ == "__main__":
    sys.exit(main())
