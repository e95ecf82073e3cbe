"""Summaries of rocprofv3 output for the layer's kernels.

Two kinds of record, both small text files meant to be kept with the code:

* duration statistics of every kernel (from ``--kernel-trace --stats
  --output-format csv``), as a Markdown table;
* HBM traffic of one kernel per launch, from two ``--pmc`` passes
  (``FETCH_SIZE``, then ``WRITE_SIZE``, each in KiB per dispatch), each scaled
  by what the same counter reads for a plain device copy of known size.  The
  record carries a digest of the library sources, so that a reader (bench.py)
  can tell whether the kernels have changed since the counters were taken.

Usage (on the output directories rocprofv3 wrote)::

    python -m mixture_experts_gemv_amd.profiling stats DIR --title T --command C --out FILE.md
    python -m mixture_experts_gemv_amd.profiling traffic --kernel k_gateup_m1 \\
        --workload gpt-oss-20b_M1 --fetch DIR --write DIR --copy-fetch DIR \\
        --copy-write DIR --copy-bytes N --command C --out FILE.json
    python -m mixture_experts_gemv_amd.profiling restamp profiles --commit C

The digest covers the code only (comments and layout removed), so a comment
edit keeps the records valid; `restamp` re-stamps records after such edits
once it has checked that the code equals that of the commit the counters
were taken at.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
COPY_KERNEL = "__amd_rocclr_copyBuffer"


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def _code_only(text: str) -> str:
    """C/C++ source with comments removed and whitespace runs collapsed, so
    that editing a comment does not change the digest of the code."""
    return " ".join(_COMMENT.sub(" ", text).split())


def source_digest() -> str:
    """sha256 over the library's kernel and ABI sources (file names and code,
    comments and layout excluded)."""
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        if not os.path.isfile(f) or not f.endswith((".hip", ".h", ".cpp", ".cc")):
            continue
        h.update(os.path.basename(f).encode() + b"\0")
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def _find(root: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(root, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {root}")
    return hits[0]


def short_name(name: str) -> str:
    """Kernel symbol without its argument list and namespace."""
    n = re.sub(r"\(.*", "", name).strip()
    n = re.sub(r"^void\s+", "", n)
    return n.replace("moe::", "")


def kernel_stats(root: str) -> list[dict]:
    """Rows of rocprofv3's kernel_stats.csv, durations in microseconds."""
    rows = []
    with open(_find(root, "kernel_stats.csv")) as fh:
        for r in csv.DictReader(fh):
            rows.append(dict(name=short_name(r["Name"]), calls=int(r["Calls"]),
                             avg_us=float(r["AverageNs"]) / 1e3, min_us=float(r["MinNs"]) / 1e3,
                             max_us=float(r["MaxNs"]) / 1e3, total_us=float(r["TotalDurationNs"]) / 1e3,
                             pct=float(r["Percentage"])))
    return rows


def counter_per_dispatch(root: str, counter: str) -> dict[str, tuple[float, int]]:
    """Mean value of `counter` per dispatch, and the dispatch count, by kernel."""
    acc: dict[str, list[float]] = {}
    with open(_find(root, "counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(short_name(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def pick(table: dict, kernel: str):
    keys = [k for k in table if kernel in k]
    if len(keys) != 1:
        raise KeyError(f"kernel {kernel!r} matches {keys} in {sorted(table)}")
    return keys[0], table[keys[0]]


def write_stats(args) -> None:
    rows = kernel_stats(args.dir)
    out = [f"# {args.title}", "", "Command:", "", "```", args.command, "```", "",
           "| kernel | calls | avg us | min us | max us | % of GPU time |",
           "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        out.append(f"| `{r['name']}` | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                   f"{r['max_us']:.2f} | {r['pct']:.1f} |")
    with open(args.out, "w") as fh:
        fh.write("\n".join(out) + "\n")


def write_traffic(args) -> None:
    fetch = counter_per_dispatch(args.fetch, "FETCH_SIZE")
    write = counter_per_dispatch(args.write, "WRITE_SIZE")
    cf = counter_per_dispatch(args.copy_fetch, "FETCH_SIZE")
    cw = counter_per_dispatch(args.copy_write, "WRITE_SIZE")
    _, (cf_kib, _) = pick(cf, COPY_KERNEL)
    _, (cw_kib, _) = pick(cw, COPY_KERNEL)
    f_factor = args.copy_bytes / (cf_kib * 1024.0)
    w_factor = args.copy_bytes / (cw_kib * 1024.0)
    name, (f_kib, nf) = pick(fetch, args.kernel)
    _, (w_kib, nw) = pick(write, args.kernel)
    rec = dict(kernel=name, workload=args.workload, source_sha256=source_digest(),
               fetch_kib_per_dispatch=f_kib, write_kib_per_dispatch=w_kib, dispatches=[nf, nw],
               copy_bytes=args.copy_bytes, copy_fetch_kib=cf_kib, copy_write_kib=cw_kib,
               fetch_factor=f_factor, write_factor=w_factor,
               fetch_bytes=f_kib * 1024.0 * f_factor, write_bytes=w_kib * 1024.0 * w_factor,
               command=args.command)
    rec["traffic_bytes"] = rec["fetch_bytes"] + rec["write_bytes"]
    with open(args.out, "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")


def load_traffic(profiles_dir: str, kernel: str, workload: str) -> dict | None:
    """The traffic record for (kernel, workload) if its sources match the tree."""
    digest = source_digest()
    for f in sorted(glob.glob(os.path.join(profiles_dir, "*.traffic.json"))):
        try:
            rec = json.load(open(f))
        except (OSError, ValueError):
            continue
        if rec.get("workload") == workload and kernel in rec.get("kernel", "") \
                and rec.get("source_sha256") == digest:
            rec["_file"] = f
            return rec
    return None


def restamp(args) -> int:
    """Give the traffic records in `args.dir` the current digest, after
    checking that every source's code (comments and layout aside) equals its
    code at `args.commit`, the commit the counters were taken at."""
    import subprocess
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in srcs:
        if not f.endswith((".hip", ".h", ".cpp", ".cc")):
            continue
        rel = os.path.relpath(f, ROOT)
        old = subprocess.run(["git", "-C", ROOT, "show", f"{args.commit}:{rel}"], capture_output=True, text=True)
        if old.returncode != 0:
            print(f"{rel}: not in {args.commit}", file=sys.stderr)
            return 1
        with open(f, encoding="utf-8") as fh:
            if _code_only(old.stdout) != _code_only(fh.read()):
                print(f"{rel}: code differs from {args.commit}; take the counters again", file=sys.stderr)
                return 1
    digest = source_digest()
    for f in sorted(glob.glob(os.path.join(args.dir, "*.traffic.json"))):
        with open(f) as fh:
            rec = json.load(fh)
        rec["source_sha256"] = digest
        with open(f, "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="python -m mixture_experts_gemv_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    for k in ("kernel", "workload", "fetch", "write", "copy-fetch", "copy-write", "command", "out"):
        t.add_argument("--" + k, required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    r = sub.add_parser("restamp")
    r.add_argument("dir")
    r.add_argument("--commit", required=True)
    args = ap.parse_args(argv)
    if args.cmd == "restamp":
        return restamp(args)
    (write_stats if args.cmd == "stats" else write_traffic)(args)
    return 0


if __name__ == "__main__":
    sys.exit(main())
