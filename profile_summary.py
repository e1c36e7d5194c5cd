"""Summaries of rocprofv3 output for the measurement record in profiles/.

  python profile_summary.py trace CSV TITLE COMMAND [--bench-json FILE]
      kernel_trace.csv -> markdown table of kernel durations (per kernel and grid),
      optionally followed by the JSON line bench.py printed in the traced run
  python profile_summary.py counters CSV [NAME_SUBSTRING]
      counter_collection.csv -> mean value per dispatch of each counter, per kernel
  python profile_summary.py mfma CSV [CSV ...] [--filter NAME]
      counter_collection.csv passes -> per kernel: MFMA busy share of SIMD cycles
      (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs), VALU and LDS
      instructions per MFMA, wait share, as a markdown table
  python profile_summary.py traffic OUT.json --kernel NAME --calib-fetch CSV --calib-write CSV
                                    --fetch CSV [CSV ...] --write CSV [CSV ...]
      HBM bytes per launch of one kernel: FETCH_SIZE and WRITE_SIZE (KiB per dispatch)
      each scaled by the factor that makes the same counter read the known size of a
      plain 1 GiB device copy (bench.py --copy-calibration), averaged over the
      given runs with equal weight per run (one run per decode batch size), and
      stamped with the hash of the kernel sources (bench.py reports it only while
      the hash matches).
"""
import argparse
import collections
import csv
import json
import sys

COPY_BYTES = 1 << 30  # bench.py --copy-calibration copies this many bytes per dispatch


def _rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def trace(path, title, command, name_filter="b12x"):
    d = collections.defaultdict(list)
    for r in _rows(path):
        name = r["Kernel_Name"]
        if name_filter not in name:
            continue
        grid = int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"])
        key = (name, grid, r["Workgroup_Size_X"], r.get("VGPR_Count", ""), r.get("Accum_VGPR_Count", ""),
               r.get("LDS_Block_Size", ""))
        d[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    out = [f"# {title}\n", f"Command (from the repository root, one MI355X):\n\n```\n{command}\n```\n",
           "Durations from rocprofv3 kernel-trace begin/end timestamps, in microseconds, per kernel and grid.\n",
           "| kernel | workgroups | threads | VGPR | AGPR | LDS B | calls | avg us | median us | min us | max us |",
           "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for k, v in sorted(d.items(), key=lambda kv: -sum(kv[1])):
        v.sort()
        name = k[0].replace("void ", "").split("(")[0]
        out.append(f"| `{name}` | {k[1]} | {k[2]} | {k[3]} | {k[4]} | {k[5]} | {len(v)} | {sum(v) / len(v):.2f} | "
                   f"{v[len(v) // 2]:.2f} | {v[0]:.2f} | {v[-1]:.2f} |")
    return "\n".join(out) + "\n"


def counter_means(path, name_filter=""):
    """{kernel name: {counter: mean per dispatch}}"""
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in _rows(path):
        name = r.get("Kernel_Name", "").replace("void ", "").split("(")[0]
        if name_filter not in name:
            continue
        acc[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return {n: {c: sum(v) / len(v) for c, v in d.items()} for n, d in acc.items()}


def _single(path, counter, name_filter):
    means = counter_means(path, name_filter)
    vals = [d[counter] for d in means.values() if counter in d]
    if len(vals) != 1:
        raise SystemExit(f"{path}: expected one kernel matching {name_filter!r} with {counter}, found {len(vals)}")
    return vals[0]


def traffic(args):
    sys.path.insert(0, ".")
    import bench
    fetch_factor = COPY_BYTES / (1024.0 * _single(args.calib_fetch, "FETCH_SIZE", args.calib_kernel))
    write_factor = COPY_BYTES / (1024.0 * _single(args.calib_write, "WRITE_SIZE", args.calib_kernel))
    if len(args.fetch) != len(args.write):
        raise SystemExit("one --write run per --fetch run")
    per_run = []
    for f, w in zip(args.fetch, args.write):
        fk = _single(f, "FETCH_SIZE", args.kernel)
        wk = _single(w, "WRITE_SIZE", args.kernel)
        per_run.append({"fetch_kib": fk, "write_kib": wk,
                        "bytes": 1024.0 * (fk * fetch_factor + wk * write_factor)})
    rec = {"kernel": args.kernel, "source_sha256": bench.kernel_source_hash(),
           "fetch_factor": round(fetch_factor, 4), "write_factor": round(write_factor, 4),
           "runs": per_run, "bytes_per_launch": round(sum(r["bytes"] for r in per_run) / len(per_run)),
           "commands": args.commands}
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


XCDS = 8          # GRBM_GUI_ACTIVE is summed over the XCDs
SIMDS = 256 * 4   # compute units x SIMDs


def mfma_table(paths, name_filter=""):
    merged = collections.defaultdict(dict)
    for p in paths:
        for name, d in counter_means(p, name_filter).items():
            merged[name].update(d)
    out = ["| kernel | MFMA busy (of SIMD cycles) | MFMA instr | VALU instr / MFMA | LDS instr / MFMA | "
           "wait cycles / wave cycles | VMEM rd instr / MFMA |", "|---|---:|---:|---:|---:|---:|---:|"]
    for name, d in sorted(merged.items()):
        def g(k):
            return d.get(k, float("nan"))
        busy = g("SQ_VALU_MFMA_BUSY_CYCLES") / (g("GRBM_GUI_ACTIVE") / XCDS * SIMDS)
        mf = g("SQ_INSTS_MFMA")
        out.append(f"| `{name}` | {100 * busy:.1f}% | {mf:.4g} | {g('SQ_INSTS_VALU') / mf:.2f} | "
                   f"{g('SQ_INSTS_LDS') / mf:.2f} | {g('SQ_WAIT_ANY') / g('SQ_WAVE_CYCLES'):.2f} | "
                   f"{g('SQ_INSTS_VMEM_RD') / mf:.2f} |")
    return "\n".join(out) + "\n"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("csv")
    t.add_argument("title")
    t.add_argument("command")
    t.add_argument("--filter", default="b12x")
    t.add_argument("--bench-json", help="the JSON line bench.py printed in the traced run, appended as is")
    c = sub.add_parser("counters")
    c.add_argument("csv")
    c.add_argument("name", nargs="?", default="")
    m = sub.add_parser("mfma")
    m.add_argument("csv", nargs="+")
    m.add_argument("--filter", default="")
    r = sub.add_parser("traffic")
    r.add_argument("out")
    r.add_argument("--kernel", required=True, help="substring of the kernel name")
    r.add_argument("--calib-kernel", default="copy", help="substring of the copy kernel's name")
    r.add_argument("--calib-fetch", required=True)
    r.add_argument("--calib-write", required=True)
    r.add_argument("--fetch", nargs="+", required=True)
    r.add_argument("--write", nargs="+", required=True)
    r.add_argument("--commands", nargs="*", default=[])
    a = ap.parse_args()
    if a.cmd == "trace":
        sys.stdout.write(trace(a.csv, a.title, a.command, a.filter))
        if a.bench_json:
            with open(a.bench_json) as f:
                line = [ln for ln in f.read().splitlines() if ln.startswith("{")][-1]
            sys.stdout.write("\nThe line bench.py printed in the same run (its own HIP-event timings):\n\n"
                             f"```json\n{line}\n```\n")
    elif a.cmd == "mfma":
        sys.stdout.write(mfma_table(a.csv, a.filter))
    elif a.cmd == "counters":
        for name, d in sorted(counter_means(a.csv, a.name).items()):
            print(name)
            for k in sorted(d):
                print(f"    {k:32s} {d[k]:.6g}")
    else:
        traffic(a)


if __name__ == "__main__":
    main()
