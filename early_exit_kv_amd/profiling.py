"""Turn rocprofv3 output into the short text summaries kept under profiles/.

    python -m early_exit_kv_amd.profiling trace <kernel_stats.csv> <out.md> "<command>"
    python -m early_exit_kv_amd.profiling traffic <fetch_counter_collection.csv>
        <write_counter_collection.csv> <kernel-name-substring> <out.json> "<fetch command>"
        "<write command>" <copy bytes>

    python -m early_exit_kv_amd.profiling counters <out.md> <counter_collection.csv> [...]
        -- "<command>" [...]

``trace`` tabulates a ``--kernel-trace --stats`` run (calls, mean and total
duration per kernel).  ``traffic`` takes two ``--pmc`` runs of the same
program, one with FETCH_SIZE and one with WRITE_SIZE (KiB per dispatch), and
scales each counter by what it reads for the largest plain copy in the same
run (the runtime's buffer-copy kernel of a known size, which must fetch and
write exactly its size), giving HBM-side bytes per launch of one kernel.  The
result carries a digest of the kernel sources so that a later reader can tell
whether the kernels have changed since the counters were taken.
``counters`` tabulates the mean per dispatch of every counter of one or more
``--pmc`` runs (instruction mix, matrix-core busy cycles, wait cycles).
"""
import csv
import hashlib
import json
import os
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_source_digest():
    """sha256 over every kernel source and header of the library."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def summarize_trace(stats_csv, out_md, command, top=16):
    rows = _rows(stats_csv)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["# rocprofv3 kernel trace summary", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | mean us | total ms | % |", "|---|---:|---:|---:|---:|"]
    for r in rows[:top]:
        name = r["Name"].replace("|", "/")
        if len(name) > 90:
            name = name[:87] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counter(rows, counter):
    """(kernel name, value KiB) per dispatch for one counter."""
    out = []
    for r in rows:
        name = r.get("Counter_Name") or r.get("counter_name")
        if name != counter:
            continue
        kname = r.get("Kernel_Name") or r.get("kernel_name") or ""
        out.append((kname, float(r.get("Counter_Value") or r.get("counter_value"))))
    return out


def _copy_factor(vals, what):
    copies = [v for k, v in vals if COPY_KERNEL in k]
    if not copies:
        raise SystemExit(f"no {COPY_KERNEL} dispatch in the {what} run")
    return copies


def summarize_traffic(fetch_csv, write_csv, kernel, out_json, cmd_fetch, cmd_write, copy_bytes):
    res = {"kernel": kernel, "source_digest": kernel_source_digest(), "copy_bytes": copy_bytes,
           "commands": {"FETCH_SIZE": cmd_fetch, "WRITE_SIZE": cmd_write}}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        vals = _counter(_rows(path), counter)
        copies = sorted(_copy_factor(vals, counter))
        big = copies[-1]
        factor = copy_bytes / (big * 1024.0)
        ks = [v for k, v in vals if kernel in k]
        if not ks:
            raise SystemExit(f"no dispatch of {kernel} in the {counter} run")
        mean_kib = sum(ks) / len(ks)
        res[counter] = {"dispatches": len(ks), "mean_kib": mean_kib, "copy_kib": big,
                        "scale": factor, "bytes_per_launch": mean_kib * 1024.0 * factor}
    res["bytes_per_launch"] = res["FETCH_SIZE"]["bytes_per_launch"] + res["WRITE_SIZE"]["bytes_per_launch"]
    with open(out_json, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")
    return res


def load_traffic(path):
    """Bytes per launch from a traffic summary, or None when it is missing or
    the kernel sources changed since it was taken."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_digest") != kernel_source_digest():
        return None
    return t.get("bytes_per_launch")


def summarize_counters(csv_paths, out_md, commands, top=12):
    """Mean value per dispatch of every counter in one or more ``--pmc`` runs,
    per kernel (the kernels with the most dispatches first)."""
    per = {}
    for path in csv_paths:
        for r in _rows(path):
            name = r.get("Counter_Name") or r.get("counter_name")
            kname = r.get("Kernel_Name") or r.get("kernel_name") or ""
            val = float(r.get("Counter_Value") or r.get("counter_value"))
            disp = r.get("Dispatch_Id") or r.get("dispatch_id") or ""
            k = per.setdefault(kname, {})
            k.setdefault(name, {}).setdefault(disp, 0.0)
            k[name][disp] += val       # (a counter reported per XCD or per SE is summed)
    counters = sorted({c for k in per.values() for c in k})
    kernels = sorted(per, key=lambda k: -max(len(v) for v in per[k].values()))[:top]
    lines = ["# rocprofv3 hardware counters, mean per dispatch", "", "Commands:", "", "```"] + list(commands) + \
            ["```", "", "| kernel | dispatches | " + " | ".join(counters) + " |",
             "|---|---:|" + "---:|" * len(counters)]
    for k in kernels:
        n = max(len(v) for v in per[k].values())
        vals = []
        for c in counters:
            d = per[k].get(c)
            vals.append(f"{sum(d.values()) / len(d):.4g}" if d else "")
        name = k.replace("|", "/")
        if len(name) > 70:
            name = name[:67] + "..."
        lines.append(f"| `{name}` | {n} | " + " | ".join(vals) + " |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    if len(sys.argv) >= 5 and sys.argv[1] == "trace":
        summarize_trace(sys.argv[2], sys.argv[3], sys.argv[4])
    elif len(sys.argv) >= 9 and sys.argv[1] == "traffic":
        r = summarize_traffic(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6], sys.argv[7],
                              int(sys.argv[8]))
        print(json.dumps(r, indent=1))
    elif len(sys.argv) >= 5 and sys.argv[1] == "counters":
        # counters <out.md> <csv> [<csv> ...] -- "<command>" ["<command>" ...]
        i = sys.argv.index("--")
        summarize_counters(sys.argv[3:i], sys.argv[2], sys.argv[i + 1:])
    else:
        print(__doc__)
        sys.exit(2)
