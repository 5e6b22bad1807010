"""Cost model of one verify step: kernel factor and overhead factor.

The decomposition follows the bottleneck analysis in besthub.dev, "SpecPilot:
AI Agent Framework Boosts Speculative Decoding 10.87x for Qwen3.8-27B",
section "Phase 0: Bottleneck Analysis": every kernel type gets a byte lower
bound, the larger of its FLOP time at 60% of the dense peak and its byte time
at 90% of the bandwidth peak; the kernel factor is the profiled step time
(summed kernel durations) over the sum of those bounds, and the overhead
factor is the measured wall-clock step time over the profiled step time.  The
acceptance factor is left out: it needs the draft model's candidate lattices,
and drafts here are synthetic.

Kernel types of this library: the weight GEMMs (all layers and the LM head),
attention (the tree-masked kernel and its split merge), the recurrent layers'
state fork and commit, and everything else (embedding, RoPE and KV write,
residual reduce, argmax reduce, path walk, KV compaction), whose algorithmic
bytes are zero in this model: their time is overhead of the decomposition.

Usage (report from a rocprofv3 kernel trace and a bench.py JSON line of the
same workload and weight storage):

    python -m tree_verification_spec_amd.costmodel --trace DIR --bench FILE [--out FILE]
"""

import argparse
import collections
import csv
import glob
import json
import os
import re
import statistics

PEAK_HBM = 8.0e12        # MI355X HBM3E, bytes/s
PEAK_BF16 = 2.5e15       # MI355X dense bf16 MFMA, FLOP/s
FLOP_EFF, BYTE_EFF = 0.6, 0.9

TYPES = ("gemm", "attention", "recurrent", "other")

_TYPE_OF = [
    (re.compile(r"\bgemm(_tall)?_kernel\b"), "gemm"),
    (re.compile(r"\battn_(combine_|stream_)?kernel\b"), "attention"),
    (re.compile(r"\blr_(fork|commit)_kernel\b"), "recurrent"),
    (re.compile(r"\b(embed|rope_kv|resid_reduce|argmax_reduce|path_walk|kv_compact)_kernel\b"),
     "other"),
]


def kernel_type(name):
    """The kernel type of a kernel name from a trace, or None for kernels
    that are not part of a verify step (weight load, conversions)."""
    for pat, t in _TYPE_OF:
        if pat.search(name):
            return t
    return None


def lower_bound(nbytes, flops):
    """Seconds: the larger of FLOP time at 60% of the bf16 peak and byte
    time at 90% of the HBM peak."""
    return max(flops / (FLOP_EFF * PEAK_BF16), nbytes / (BYTE_EFF * PEAK_HBM))


def weight_bytes(rows, cols, fmt):
    """Stored bytes of one [rows, cols] matrix: 2 per bf16 weight, W12
    tiles (800 bytes per 512 weights) or the 8-bit view (1 byte a weight),
    each W12 format plus one base-exponent byte per row."""
    if fmt in ("w12", "w12_lowp"):
        return rows * cols * 800 / 512 + rows
    if fmt == "w8":
        return rows * cols + rows
    return rows * cols * 2


def type_bounds(specs, cfg, req_rows, req_ctx, fmt):
    """Algorithmic bytes and FLOPs per kernel type for one verify step.

    specs: the (name, shape, kind) tensor list of the model; req_rows: rows
    (root + drafts) per request; req_ctx: committed tokens per request.
    gemm: every weight matrix but the embedding once, 2 FLOPs per weight and
    row.  attention: each request's committed K/V once plus the pass's new
    K/V; 4 FLOPs per (query head, head dim, row, visible key).  recurrent:
    each request's states read and written once; 4 FLOPs per state element
    and row.  other: nothing algorithmic."""
    mats = [s for n, s, k in specs if k == "mat" and n != "embed"]
    n_params = sum(r * c for r, c in mats)
    wbytes = sum(weight_bytes(r, c, fmt) for r, c in mats)
    n_attn = cfg["layer_kinds"].count("A")
    n_lr = cfg["layer_kinds"].count("L")
    kv_pos = n_attn * cfg["n_kv_heads"] * cfg["head_dim"] * 2 * 2
    R = sum(req_rows)
    vis = sum(r * (c + r) for r, c in zip(req_rows, req_ctx))
    state_elems = n_lr * cfg["d_model"] * cfg["lr_state"]  # per request, fp32
    return {
        "gemm": (wbytes, 2.0 * n_params * R),
        "attention": (sum(req_ctx) * kv_pos + R * kv_pos,
                      4.0 * cfg["n_heads"] * cfg["head_dim"] * n_attn * vis),
        "recurrent": (2.0 * 4 * state_elems * len(req_rows), 4.0 * state_elems * R),
        "other": (0.0, 0.0),
    }


def factors(measured_us, bound_us, wall_us):
    """Kernel factor = profiled step time / summed lower bounds; overhead
    factor = wall step time / profiled step time.  Their product is the
    wall step time over the summed lower bounds."""
    profiled = sum(measured_us.values())
    bound = sum(bound_us.values())
    return {
        "profiled_us": profiled,
        "bound_us": bound,
        "wall_us": wall_us,
        "kernel_factor": profiled / bound,
        "overhead_factor": wall_us / profiled,
        "total_factor": wall_us / bound,
    }


# ------------------------------------------------------------ trace parsing

def _pass_rows(row):
    """Rows of the pass an embedding launch belongs to: the embedding kernel
    runs one 256-thread workgroup per row (and chunk of columns, in y)."""
    return int(row.get("Grid_Size_X", 0)) // 256


def verify_steps(rows, n_rows):
    """Split kernel-trace rows (sorted by start) into verify steps: from an
    embedding launch to the next one, keeping the steps of exactly `n_rows`
    rows that contain the accepted-path walk (this leaves out prefill chunks,
    which have no walk, and passes of other sizes such as the AR run).  A
    step's kernels include its commit (KV compaction, recurrent state
    commit), which runs before the next pass's embedding.  Returns a list of
    row lists."""
    steps, cur, cur_rows = [], None, 0
    for r in rows:
        n = r["Kernel_Name"]
        if "embed_kernel" in n:
            if cur is not None:
                steps.append((cur_rows, cur))
            cur, cur_rows = [], _pass_rows(r)
        if cur is not None and kernel_type(n) is not None:
            cur.append(r)
    if cur:
        steps.append((cur_rows, cur))
    return [st for nr, st in steps
            if nr == n_rows and any("path_walk_kernel" in r["Kernel_Name"] for r in st)]


def _dur_us(r):
    return (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3


def steps_from_trace(rows, n_rows):
    """Per verify step (see verify_steps) the summed kernel time of each
    kernel type, as a list of {type: microseconds}."""
    out = []
    for st in verify_steps(rows, n_rows):
        per = collections.Counter()
        for r in st:
            per[kernel_type(r["Kernel_Name"])] += _dur_us(r)
        out.append(per)
    return out


def kernel_table(steps):
    """Per kernel (name and grid size) over the given verify steps: launches
    per step, mean microseconds per step and per launch, sorted by time."""
    acc = collections.defaultdict(list)
    for st in steps:
        for r in st:
            acc[(r["Kernel_Name"], int(r.get("Grid_Size_X", 0)),
                 int(r.get("Grid_Size_Y", 1) or 1))].append(_dur_us(r))
    n = len(steps)
    out = []
    for (name, gx, gy), d in acc.items():
        out.append(dict(kernel=name, grid=(gx, gy), per_step=len(d) / n,
                        us_per_step=sum(d) / n, avg_us=statistics.mean(d),
                        median_us=statistics.median(d)))
    out.sort(key=lambda k: -k["us_per_step"])
    return out


def report(trace_dir, bench):
    """Markdown report and numbers for one workload: per-type measured time
    (mean over the trace's verify steps), lower bounds (from the bench's
    per-step algorithmic bytes and FLOPs) and the two factors."""
    f = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not f:
        raise SystemExit(f"no kernel trace under {trace_dir}")
    rows = sorted(csv.DictReader(open(f[0])), key=lambda r: int(r["Start_Timestamp"]))
    cm = bench["cost_model"]
    raw = verify_steps(rows, cm["rows"])
    if not raw:
        raise SystemExit("no verify steps with the bench's row count in the trace")
    steps = steps_from_trace(rows, cm["rows"])
    measured = {t: statistics.mean(s.get(t, 0.0) for s in steps) for t in TYPES}
    bound = {t: cm["types"][t]["bound_us"] for t in TYPES}
    fac = factors(measured, bound, 1e3 * bench["ms_per_step"])
    lines = [
        f"# Cost model: {bench['config']['workload']} ({bench['config'].get('weights')} weights)",
        "",
        f"{len(steps)} verify steps in the trace; lower bounds per step from the "
        f"benchmark's algorithmic bytes and FLOPs (FLOPs at {FLOP_EFF:.0%} of "
        f"{PEAK_BF16 / 1e15:.1f} PFLOP/s, bytes at {BYTE_EFF:.0%} of "
        f"{PEAK_HBM / 1e12:.0f} TB/s).",
        "",
        "| kernel type | measured us per step | bytes per step | FLOPs per step | lower bound us | efficiency |",
        "|---|---|---|---|---|---|",
    ]
    for t in TYPES:
        ty = cm["types"][t]
        eff = bound[t] / measured[t] if measured[t] > 0 else float("nan")
        lines.append(f"| {t} | {measured[t]:.1f} | {ty['bytes']:.4g} | {ty['flops']:.4g} | "
                     f"{bound[t]:.1f} | {eff:.3f} |")
    lines += [
        "",
        f"- profiled step time (summed kernel durations): {fac['profiled_us']:.1f} us",
        f"- summed lower bounds: {fac['bound_us']:.1f} us",
        f"- wall step time (benchmark, unprofiled): {fac['wall_us']:.1f} us",
        f"- kernel factor: {fac['kernel_factor']:.3f}",
        f"- overhead factor: {fac['overhead_factor']:.3f}",
        f"- kernel factor x overhead factor: {fac['total_factor']:.3f}",
        f"- largest factor: {'kernel' if fac['kernel_factor'] >= fac['overhead_factor'] else 'overhead'}",
        "",
        "Kernels of a verify step (mean over the steps above; grid in threads):",
        "",
        "| kernel | grid x, y | launches per step | us per step | share | mean us per launch | median us |",
        "|---|---|---|---|---|---|---|",
    ]
    kt = kernel_table(raw)
    stats = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    for k in kt:
        lines.append(f"| `{k['kernel']}` | {k['grid'][0]}, {k['grid'][1]} | "
                     f"{k['per_step']:.2f} | {k['us_per_step']:.1f} | "
                     f"{k['us_per_step'] / fac['profiled_us']:.1%} | {k['avg_us']:.2f} | "
                     f"{k['median_us']:.2f} |")
    if stats:
        # rocprofv3 --stats over the whole traced run (every pass: prefill,
        # the AR reference, verify steps), the largest total times
        rows_s = sorted(csv.DictReader(open(stats[0])), key=lambda r: -float(r["TotalDurationNs"]))
        lines += ["", "rocprofv3 --stats of the traced run (all passes), by total time:", "",
                  "| kernel | calls | total ms | average us | min us | max us |",
                  "|---|---|---|---|---|---|"]
        for r in rows_s[:16]:
            lines.append(f"| `{r['Name']}` | {r['Calls']} | {float(r['TotalDurationNs']) / 1e6:.2f} | "
                         f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                         f"{float(r['MaxNs']) / 1e3:.2f} |")
    return "\n".join(lines) + "\n", dict(measured=measured, bound=bound, kernels=kt, **fac)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--trace", required=True, help="rocprofv3 kernel-trace output directory")
    ap.add_argument("--bench", required=True, help="file holding bench.py's JSON line")
    ap.add_argument("--out", default=None)
    ap.add_argument("--commands", default=None,
                    help="file holding the commands that produced the trace and the JSON line")
    a = ap.parse_args()
    bench = None
    for line in open(a.bench):
        line = line.strip()
        if line.startswith("{") and '"cost_model"' in line:
            bench = json.loads(line)
    if bench is None:
        raise SystemExit(f"no bench JSON line with a cost_model in {a.bench}")
    text, _ = report(a.trace, bench)
    if a.commands:
        head, rest = text.split("\n", 1)
        text = (head + "\n\nCommands (from the repository root, on one MI355X):\n\n```\n" +
                open(a.commands).read().strip() + "\n```\n" + rest)
    if a.out:
        with open(a.out, "w") as fh:
            fh.write(text)
    print(text, end="")


if __name__ == "__main__":
    main()
