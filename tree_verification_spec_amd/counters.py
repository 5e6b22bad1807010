"""Summaries of rocprofv3 hardware-counter passes over benchmark runs.

traffic: HBM bytes per launch of one kernel from a FETCH_SIZE pass and a
WRITE_SIZE pass (KiB per dispatch), each scaled by what the same counter
reads for a plain elementwise copy of known size run first in the same
process (bench.py --copy-probe-bytes N: dst = -src over N bytes, which
reads N and writes N bytes).  The summary records a hash of the kernel's
sources, so that a reader of it (bench.py) can tell when the kernel has
changed since the counters were taken.

mfma: per kernel (name and grid size) the matrix-core busy fraction
(rocprofv3's derived MfmaUtil: MFMA-busy cycles over GPU-active cycles times
the SIMD count) and the bf16 MFMA FLOPs per launch, from one pass of
`--pmc MfmaUtil MfmaFlopsBF16`.

    python -m tree_verification_spec_amd.counters traffic --fetch DIR --write DIR \\
        --kernel REGEX [--grid N] --copy-bytes N --alg-bytes N --title TEXT \\
        --commands FILE [--out FILE]
    python -m tree_verification_spec_amd.counters mfma --dir DIR [--kernel REGEX] \\
        --title TEXT --commands FILE [--out FILE]
"""

import argparse
import collections
import csv
import glob
import hashlib
import os
import re
import statistics

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = [os.path.join(ROOT, "tree_verification_spec_amd", "csrc", f)
                  for f in ("gemm.hip", "common.h", "kernels.h", "w12.h")]


def kernel_source_hash(paths=KERNEL_SOURCES):
    """First 16 hex digits of the SHA-256 of the GEMM kernel's sources."""
    h = hashlib.sha256()
    for f in paths:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_summary_fields(path):
    """The `- key: value` lines of a summary written by `traffic`."""
    kv = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("- ") and ": " in line:
                k, v = line[2:].strip().split(": ", 1)
                kv[k.strip("`")] = v.strip().strip("`")
    return kv


def _counter_rows(d):
    f = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return list(csv.DictReader(open(f[0])))


def _grid(r):
    for k in ("Grid_Size", "Grid_Size_X"):
        if k in r and r[k]:
            return int(r[k])
    return 0


def per_dispatch(rows, counter):
    """{dispatch id: (kernel name, grid size, value)} of one counter."""
    out = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        d = r.get("Dispatch_Id") or r.get("Correlation_Id")
        name, g, v = r["Kernel_Name"], _grid(r), float(r["Counter_Value"])
        if d in out:  # one row per counter instance: sum them
            name0, g0, v0 = out[d]
            out[d] = (name0, g0, v0 + v)
        else:
            out[d] = (name, g, v)
    return out


def traffic(fetch_dir, write_dir, kernel, grid, copy_bytes):
    """Per counter: (kernel mean KiB per dispatch, dispatches, copy KiB,
    scale, kernel bytes per dispatch after scaling)."""
    pat = re.compile(kernel)
    res = {}
    for ctr, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        disp = per_dispatch(_counter_rows(d), ctr)
        k = [v for n, g, v in disp.values() if pat.search(n) and (not grid or g == grid)]
        cp = [v for n, g, v in disp.values() if "neg_kernel" in n]
        if len(cp) != 1 or not k:
            raise SystemExit(f"{ctr}: {len(k)} kernel dispatches, {len(cp)} copy dispatches")
        scale = cp[0] / (copy_bytes / 1024)
        m = statistics.mean(k)
        res[ctr] = (m, len(k), cp[0], scale, m * 1024 / scale)
    return res


def traffic_report(res, title, commands, alg_bytes, copy_bytes):
    tot = int(round(res["FETCH_SIZE"][4] + res["WRITE_SIZE"][4]))
    lines = [
        f"# {title}: HBM traffic counters", "",
        "Two counter passes over a short run of the benchmark, each first running one",
        f"elementwise copy (dst = -src) of {copy_bytes} bytes (read {copy_bytes}, write",
        f"{copy_bytes}) whose counter readings give the scale factor.", "",
        "Commands (from the repository root, on one MI355X):", "", "```",
        commands.strip(), "```", "",
        "| counter | kernel mean per dispatch (KiB) | dispatches | copy probe (KiB) | "
        "scale (copy reading / true KiB) | kernel bytes after scaling |",
        "|---|---|---|---|---|---|",
    ]
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        m, n, c, s, b = res[ctr]
        lines.append(f"| {ctr} | {m:.1f} | {n} | {c:.1f} | {s:.4f} | {int(round(b))} |")
    lines += [
        "", f"Algorithmic bytes per launch: {alg_bytes:,}; measured over algorithmic: "
            f"{tot / alg_bytes:.4f}.", "",
        f"- traffic_bytes_per_launch: {tot}",
        f"- algorithmic_bytes_per_launch: {alg_bytes}",
        f"- kernel_source_sha256_16: {kernel_source_hash()}",
        "- kernel_sources: " + ", ".join(os.path.relpath(p, ROOT) for p in KERNEL_SOURCES),
    ]
    return "\n".join(lines) + "\n"


def mfma(d, kernel=None):
    """Per (kernel, grid): dispatches, mean MfmaUtil (%) and mean bf16 MFMA
    FLOPs per dispatch, sorted by FLOPs."""
    rows = _counter_rows(d)
    util = per_dispatch(rows, "MfmaUtil")
    flops = per_dispatch(rows, "MfmaFlopsBF16")
    pat = re.compile(kernel) if kernel else None
    acc = collections.defaultdict(lambda: ([], []))
    for did, (n, g, u) in util.items():
        if pat and not pat.search(n):
            continue
        acc[(n, g)][0].append(u)
        acc[(n, g)][1].append(flops.get(did, (n, g, 0.0))[2])
    out = [dict(kernel=n, grid=g, n=len(u), util=statistics.mean(u),
                flops=statistics.mean(f)) for (n, g), (u, f) in acc.items()]
    out.sort(key=lambda k: -k["flops"] * k["n"])
    return out


def mfma_report(tab, title, commands):
    lines = [
        f"# {title}: matrix-core utilisation", "",
        "One counter pass (`MfmaUtil`: MFMA-busy cycles over GPU-active cycles x SIMD "
        "count, in percent; `MfmaFlopsBF16`: bf16 MFMA FLOPs per dispatch).", "",
        "Commands (from the repository root, on one MI355X):", "", "```",
        commands.strip(), "```", "",
        "| kernel | grid (threads) | dispatches | MfmaUtil % | bf16 MFMA GFLOP per dispatch |",
        "|---|---|---|---|---|",
    ]
    for k in tab:
        lines.append(f"| `{k['kernel']}` | {k['grid']} | {k['n']} | {k['util']:.2f} | "
                     f"{k['flops'] / 1e9:.3f} |")
    return "\n".join(lines) + "\n"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True, help="regex on the kernel name")
    t.add_argument("--grid", type=int, default=0, help="grid size in threads (0: any)")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--alg-bytes", type=int, required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--dir", required=True)
    m.add_argument("--kernel", default=None)
    for p in (t, m):
        p.add_argument("--title", required=True)
        p.add_argument("--commands", required=True, help="file holding the commands run")
        p.add_argument("--out", default=None)
    a = ap.parse_args()
    commands = open(a.commands).read()
    if a.cmd == "traffic":
        res = traffic(a.fetch, a.write, a.kernel, a.grid, a.copy_bytes)
        text = traffic_report(res, a.title, commands, a.alg_bytes, a.copy_bytes)
    else:
        text = mfma_report(mfma(a.dir, a.kernel), a.title, commands)
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text)
    print(text, end="")


if __name__ == "__main__":
    main()
