"""Benchmark of the speculative-decoding verify step on one MI355X.

Default workload (the headline): 8B-shaped dense decoder (36 layers,
d=4096, 32/8 GQA heads, FFN 12288, vocab 151936, bf16 weights, random init,
stored as W12: lossless 12-bit tiles whose GEMM results are bitwise those
of bf16 storage; --weights native keeps bf16 tiles),
2048-token random prompt, batch 1, chain drafts of K=16 tokens synthesised
from the target's own greedy continuation with per-position match
probability alpha (0.7 headline; 0.5 and 0.9 reported too).  A step is one
spec_verify + spec_commit.  --workload selects the other measured
workloads: a 64-node best-first tree at a 4096-token prompt, 32 batched
requests (contexts 512..4096, K=8, alpha 0.4..0.9 per request) verified in
one fused pass per step, and the 27B-shaped hybrid with 32-node trees.

Reported: accepted tokens/s (emitted tokens over the summed wall time of
the verify + commit calls, inputs resident in HBM; host draft synthesis
excluded), the byte lower bound of a step (max(FLOPs at 60% of 2.5 PFLOP/s,
bytes at 90% of 8 TB/s, weights counted in their stored format)) and the
fraction of it reached, the GPU
autoregressive rate (K=0, same library) and, for the dominant kernel (the
FFN gate/up GEMM), algorithmic GB/s from per-launch HIP events against the
8 TB/s HBM peak.  The CPU oracle's AR decode rate on the same model is
timed on a bounded sample as a reported baseline.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # MI355X HBM3E, bytes/s
PEAK_BF16 = 2.5e15         # MI355X dense bf16 MFMA, FLOP/s

WORKLOADS = ("dense8b_chain", "dense8b_tree", "dense8b_batched", "hybrid27b_tree")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def step_bounds(cfg, req_rows, req_ctx, fmt):
    """Algorithmic bytes, FLOPs and lower-bound seconds of one verify step,
    and the per-kernel-type (bytes, FLOPs): weights once (in their stored
    format), every request's committed KV once, the pass's new KV, the
    recurrent states read once and committed once."""
    import synth
    from tree_verification_spec_amd import costmodel
    types = costmodel.type_bounds(synth.tensor_specs(cfg), cfg, req_rows, req_ctx, fmt)
    nbytes = sum(b for b, _ in types.values())
    flops = sum(f for _, f in types.values())
    return nbytes, flops, costmodel.lower_bound(nbytes, flops), types


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="dense8b_chain", choices=WORKLOADS)
    ap.add_argument("--alpha", type=float, default=None)
    ap.add_argument("--weights", default=None, choices=("w12", "native", "w12_lowp"),
                    help="weight storage: W12 (lossless 12-bit, bitwise-identical "
                         "results) or the model's bf16; default: the faster of the two "
                         "for the workload (W12 up to 40 rows per pass, bf16 above)")
    ap.add_argument("--policy", default="fixed", choices=("fixed", "budget"),
                    help="batched workload: fixed K drafts per request, or per-step draft "
                         "lengths of 8/12/16 from each request's acceptance so far under a "
                         "shared budget of batch x K draft nodes")
    ap.add_argument("--two-level", default=None, metavar="K1,K2",
                    help="chain workloads: two-level verification steps (a pass on the "
                         "8-bit weight view over K1 drafts gives a candidate chain, the "
                         "drafter continues K2 positions, one exact pass verifies all)")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=64)
    ap.add_argument("--ref-len", type=int, default=0,
                    help="tokens of the GPU AR reference run (0: enough for the steps)")
    ap.add_argument("--copy-probe-bytes", type=int, default=0,
                    help="first run one elementwise copy (dst = -src) of this many "
                         "bytes (the known-size kernel that scales HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: the verification path runs on one GPU; --gpus N with "
              "N > 1 is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    from tree_verification_spec_amd import Engine, costmodel
    import tree_verification_spec_amd as L

    if args.copy_probe_bytes:
        n = args.copy_probe_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)        # an elementwise kernel: reads n*4, writes n*4
        torch.cuda.synchronize()
        del src, dst
        log(f"copy probe: {4 * n} bytes")

    w = synth.workload(args.workload)
    cfg = synth.model_config(w["model"])
    if args.weights is None:
        rows = w["K"] + 1 if args.workload != "dense8b_batched" else w["batch"] * (w["K"] + 1)
        args.weights = "w12" if rows <= 40 else "native"
    V, K, idx = cfg["vocab"], w["K"], w["index"]
    batched = args.workload == "dense8b_batched"
    tree = w["draft"] == "tree"
    if batched:
        B = w["batch"]
        ctx0, alphas = synth.batched_mix(B, w["ctx_lo"], w["ctx_hi"], w["alpha_lo"],
                                         w["alpha_hi"])
        prompts = [synth.prompt_tokens(V, int(ctx0[r]), idx, r) for r in range(B)]
        alpha_main = None
    else:
        B = 1
        alphas = None
        prompts = [synth.prompt_tokens(V, w["prompt"], idx)]
        alpha_main = args.alpha if args.alpha is not None else w["alpha"]
    sweep_alphas = [] if (args.no_sweep or batched or tree) else \
        [a for a in w.get("alphas", ()) if abs(a - alpha_main) > 1e-9]
    # reference length: enough tokens for every run's expected acceptance
    planned = batched and args.policy == "budget"
    two = tuple(int(x) for x in args.two_level.split(",")) if args.two_level else None
    if two and (batched or tree):
        print("bench.py: --two-level is for the chain workload", file=sys.stderr)
        sys.exit(2)
    if two:
        args.weights = "w12_lowp"
    choices, min_prob, decay = (8, 12, 16), 0.05, 0.9
    budget = B * K
    depth = w.get("max_depth", 8) if tree else (max(choices) if planned else K)
    if two:
        depth = two[0] + two[1] + 1
    runs = [(alpha_main if not batched else 0.9, args.warmup + args.steps),
            (alpha_main if not batched else 0.9, max(10, args.steps // 3) + 2)]
    runs += [(a, max(20, args.steps // 2) + 4) for a in sweep_alphas]
    need = max(synth.expected_tokens_per_step(a, depth) * n for a, n in runs)
    ref_len = args.ref_len or min(int(need * 1.5) + 64, (depth + 1) *
                                  max(n for _, n in runs) + 8)

    t0 = time.time()
    W = synth.make_weights(cfg)
    log(f"weights generated in {time.time() - t0:.1f}s")
    max_ctx = max(len(p) for p in prompts) + ref_len + 2 * (depth + 1)
    eng = Engine(cfg, device=0, max_requests=B, max_ctx=max_ctx,
                 max_nodes=(max(choices) if planned else K) + 1,
                 max_rows=B * ((depth if two else K) + 1), prefill_chunk=512,
                 weight_format=args.weights)
    t0 = time.time()
    eng.load_weights([W[n] for n, _, _ in synth.tensor_specs(cfg)])
    log(f"weights loaded in {time.time() - t0:.1f}s")

    # ---- GPU autoregressive reference (K = 0): continuations + AR rate
    sync = torch.cuda.synchronize
    t0 = time.time()
    S = [[eng.prefill(r, prompts[r])] for r in range(B)]
    sync()
    log(f"prefill of {sum(len(p) for p in prompts)} tokens in {time.time() - t0:.1f}s")
    t_ar = 0.0
    for t in range(ref_len - 1):
        a = time.perf_counter()
        paths, bonus = eng.verify(list(range(B)), [[]] * B, [[]] * B)
        eng.commit(list(range(B)), [[]] * B, bonus)
        sync()
        t_ar += time.perf_counter() - a
        for r in range(B):
            S[r].append(bonus[r])
    for r in range(B):
        eng.release(r)
    S = [np.array(s, np.int32) for s in S]
    ar_tps = B * (ref_len - 1) / t_ar
    log(f"GPU AR: {ref_len - 1} tokens x {B} requests, {ar_tps:.1f} tok/s")

    def drafts_for(r, g, step, alpha, k):
        if tree:
            return synth.tree_drafts(S[r], g, k, w["branching"], w["max_depth"], alpha, V,
                                     idx, r, step)
        return synth.chain_drafts(S[r], g, k, alpha, V, idx, r, step)

    def run(alpha, steps, warmup, timing_cls=0):
        slots = list(range(B))  # the reference run released them
        for r in range(B):
            eng.prefill(slots[r], prompts[r])
        g = [1] * B
        tot, toks, mism, lbs, lbs_b, dev_ms, types = 0.0, 0, 0, [], [], [], []
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        al = [float(a) for a in alphas] if batched else [alpha] * B
        succ, fail = [0.0] * B, [0.0] * B
        for it in range(warmup + steps):
            timed = it >= warmup
            if timed and it == warmup and timing_cls:
                eng.timing(timing_cls)
                eng.timing_read()
            t_plan = time.perf_counter()
            lens = (L.spec_plan_drafts(succ, fail, choices, min_prob, budget) if planned
                    else [K] * B)
            t_plan = time.perf_counter() - t_plan
            t_lp = 0.0
            if two:
                # low-precision round (timed), then the drafter's continuation
                # from the candidate chain's end (host synthesis, untimed)
                d1 = [drafts_for(r, g[r], it, al[r], two[0]) for r in range(B)]
                sync()
                a = time.perf_counter()
                ev0.record(eng.stream)
                lp_paths, lp_bonus = eng.verify(slots, [d[0] for d in d1], [d[1] for d in d1],
                                                lowp=True)
                t_lp = time.perf_counter() - a
                dr = []
                for r in range(B):
                    cand = [int(d1[r][0][p]) for p in lp_paths[r]] + [lp_bonus[r]]
                    cont, _ = synth.chain_drafts(S[r], g[r] + len(cand), two[1], al[r], V,
                                                 idx + 50, r, it)
                    ch = np.array(cand + [int(t) for t in cont], np.int32)
                    dr.append((ch, np.arange(-1, len(ch) - 1, dtype=np.int32)))
                lens = [len(d[0]) for d in dr]
                lp_rows = [two[0] + 1] * B
            else:
                dr = [drafts_for(r, g[r], it, al[r], lens[r]) for r in range(B)]
            ctx = [eng.state(slots[r])[0] for r in range(B)]
            sync()
            a = time.perf_counter()
            if not two:
                ev0.record(eng.stream)
            paths, bonus = eng.verify(slots, [d[0] for d in dr], [d[1] for d in dr])
            keep, roots, n_new = [], [], []
            for r in range(B):
                emitted = [int(dr[r][0][p]) for p in paths[r]] + [bonus[r]]
                n_ok = 0
                for j, tk in enumerate(emitted):
                    if g[r] + j >= len(S[r]) or tk != S[r][g[r] + j]:
                        break
                    n_ok += 1
                if n_ok < len(emitted) and g[r] + n_ok < len(S[r]):
                    # token forcing: keep the run aligned with the reference
                    kp = paths[r][:n_ok] if n_ok < len(paths[r]) else paths[r]
                    keep.append(kp)
                    roots.append(int(S[r][g[r] + n_ok]))
                    n_new.append(len(kp) + 1)
                    mism += 1
                else:
                    keep.append(paths[r])
                    roots.append(bonus[r])
                    n_new.append(len(emitted))
            eng.commit(slots, keep, roots)
            ev1.record(eng.stream)
            sync()
            dt = time.perf_counter() - a + t_lp
            if planned:
                t_upd = time.perf_counter()
                succ, fail = L.spec_acceptance_update(lens, [len(p) for p in paths], decay,
                                                      succ, fail)
                dt += t_plan + time.perf_counter() - t_upd
            if timed:
                tot += dt
                toks += sum(n_new)
                dev_ms.append(ev0.elapsed_time(ev1))
                nb, fl, lb, ty = step_bounds(cfg, [k + 1 for k in lens], ctx, args.weights)
                if two:  # the low-precision pass reads the 8-bit view
                    nb2, fl2, _, ty2 = step_bounds(cfg, lp_rows, ctx, "w8")
                    nb, fl = nb + nb2, fl + fl2
                    lb = costmodel.lower_bound(nb, fl)
                    ty = {t: (ty[t][0] + ty2[t][0], ty[t][1] + ty2[t][1]) for t in ty}
                lbs.append(lb)
                lbs_b.append(nb)
                types.append(ty)
            for r in range(B):
                g[r] += n_new[r]
        kt = None
        if timing_cls:
            kt = eng.timing_read()
            eng.timing(0)
        for r in range(B):
            eng.release(slots[r])
        return dict(tps=toks / tot, ms=1e3 * tot / steps, toks=toks,
                    tok_per_step=toks / steps, mism=mism,
                    dev_ms=float(np.median(dev_ms)),
                    dev_pct=[float(x) for x in np.percentile(dev_ms, [10, 50, 90])],
                    lb_ms=1e3 * float(np.mean(lbs)),
                    bytes=float(np.mean(lbs_b)), ktime=kt,
                    types={t: (float(np.mean([ty[t][0] for ty in types])),
                               float(np.mean([ty[t][1] for ty in types])))
                           for t in types[0]})

    res = run(alpha_main, args.steps, args.warmup)
    log(f"{args.workload} alpha={alpha_main}: {res}")
    # the dominant kernel's launch times: each gate/up launch records its own
    # start and end in a HIP event pair (extended launch; passes of this run
    # are launched kernel by kernel, without graph replay)
    rl = run(alpha_main, max(10, args.steps // 3), 2, timing_cls=1)
    log(f"timed launches: {rl}")
    sweep = {}
    for al in sweep_alphas:
        r = run(al, max(20, args.steps // 2), 4)
        sweep[str(al)] = dict(tokens_per_s=round(r["tps"], 1),
                              tokens_per_step=round(r["tok_per_step"], 3),
                              lb_frac=round(r["lb_ms"] / r["dev_ms"], 4))
        log(f"alpha={al}: {r}")
    if not batched:
        sweep[str(alpha_main)] = dict(tokens_per_s=round(res["tps"], 1),
                                      tokens_per_step=round(res["tok_per_step"], 3),
                                      lb_frac=round(res["lb_ms"] / res["dev_ms"], 4))

    # roofline of the dominant kernel: FFN gate/up GEMM, weights streamed once
    # per launch (passes of more than 128 rows launch it once per 128 rows)
    gu_bytes = costmodel.weight_bytes(2 * cfg["ffn_dim"], cfg["d_model"], args.weights)
    k_ms, k_n = rl["ktime"]
    k_avg_s = k_ms / 1e3 / max(1, k_n)
    achieved = gu_bytes / k_avg_s / 1e9

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, W, args.cpu_tokens)

    if batched:
        desc = ("8B-shaped dense decoder, 32 requests (contexts 512..4096 in 16-token "
                "pages), chain drafts K=8, alpha 0.4..0.9 per request, one fused "
                "verify per step")
        if planned:
            desc += (", draft lengths planned per step (8/12/16 by acceptance, shared "
                     f"budget of {budget} draft nodes)")
    elif two:
        desc = ("8B-shaped dense decoder, 2048-token prompt, two-level verification: "
                f"{two[0]} drafts through the 8-bit weight view, candidate chain + "
                f"{two[1]} continuation drafts through the exact pass, alpha=%.1f, batch 1"
                % alpha_main)
    elif tree:
        model = ("8B-shaped dense decoder" if w["model"] == "dense8b" else
                 "27B-shaped hybrid (48 recurrent + 16 attention layers)")
        desc = (f"{model}, {w['prompt']}-token prompt, best-first draft tree of {K} "
                f"nodes (depth <= {w['max_depth']}), alpha={alpha_main} on the main "
                f"path, batch 1")
    else:
        desc = ("8B-shaped dense decoder, 2048-token prompt, chain draft K=16, "
                "alpha=%.1f, batch 1" % alpha_main)
    out = {
        "metric": "accepted tokens/s at batch 1 + verify-step HBM GB/s vs byte lower bound",
        "value": round(res["tps"], 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (random-init weights N(0,0.02), uniform random prompt, "
                "drafts from the target's greedy continuation)",
        "config": {"workload": desc, "name": args.workload, "batch": B, "draft_K": K,
                   "alpha": alpha_main, "prompt": None if batched else w["prompt"],
                   "weights": args.weights,
                   "policy": (f"budget {budget}, lengths {list(choices)}, min_prob "
                              f"{min_prob}, decay {decay}") if planned else "fixed"},
        "verify_step": {
            "device_ms_median": round(res["dev_ms"], 4),
            "byte_lower_bound_ms": round(res["lb_ms"], 4),
            "lb_frac": round(res["lb_ms"] / res["dev_ms"], 4),
            "algorithmic_GBps": round(res["bytes"] / (res["dev_ms"] / 1e3) / 1e9, 1),
            "device_ms_p10_p50_p90": [round(x, 4) for x in res["dev_pct"]],
            "tokens_per_step": round(res["tok_per_step"], 3),
            "forced_mismatches": res["mism"],
        },
        "ar_tokens_per_s": round(ar_tps, 2),
        "speedup_over_ar": round(res["tps"] / ar_tps, 3),
        "alpha_sweep": sweep,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(achieved / (PEAK_HBM / 1e9), 4),
                     "traffic": (measured_traffic(args.weights)
                                 if args.workload == "dense8b_chain" else None),
                     "kernel": "FFN gate/up GEMM + SwiGLU (%.1f MB of %s weights per launch)"
                               % (gu_bytes / 1e6, "W12" if args.weights == "w12" else "bf16"),
                     "launches": k_n, "avg_launch_us": round(k_avg_s * 1e6, 2)},
        "cpu_baseline": cpu,
        # per-kernel-type lower bounds of the mean step (the cost model's
        # kernel and overhead factors need a kernel trace of the same run
        # shape: python -m tree_verification_spec_amd.costmodel)
        "cost_model": {
            "rows": B * (K + 1),
            "types": {t: {"bytes": b, "flops": f,
                          "bound_us": round(1e6 * costmodel.lower_bound(b, f), 2)}
                      for t, (b, f) in res["types"].items()},
        },
    }
    eng.close()
    print(json.dumps(out), flush=True)


TRAFFIC_FILES = {
    "native": os.path.join(ROOT, "profiles", "gemm_gateup_swiglu_bf16_dense8b_chain_k16_traffic.md"),
    "w12": os.path.join(ROOT, "profiles", "gemm_gateup_swiglu_w12_dense8b_chain_k16_traffic.md"),
}
TRAFFIC_SOURCES = [os.path.join(ROOT, "tree_verification_spec_amd", "csrc", f)
                   for f in ("gemm.hip", "common.h", "kernels.h", "w12.h")]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(fmt):
    """HBM bytes per gate/up launch from the committed counter summary for
    this weight format (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of
    known size), or None when the kernel sources changed since the counters
    were taken."""
    try:
        kv = {}
        with open(TRAFFIC_FILES[fmt]) as fh:
            for line in fh:
                if line.startswith("- ") and ": " in line:
                    k, v = line[2:].strip().split(": ", 1)
                    kv[k.strip("`")] = v.strip().strip("`")
        if kv.get("kernel_source_sha256_16") != kernel_source_hash():
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(cfg, W, n_tok):
    """The oracle's AR decode rate on the same model (fp32 numpy on the host
    cores), after a short prompt; weight widening is done before the timed
    tokens."""
    import numpy as np
    import synth
    from oracle import Model
    cores = len(os.sched_getaffinity(0))
    m = Model(cfg, W, max_pos=4096)
    st = m.new_state()
    t0 = time.time()
    lg = m.prefill(st, synth.prompt_tokens(cfg["vocab"], 32, 99))
    log(f"cpu oracle: prefill+widen {time.time() - t0:.1f}s")
    tok = int(np.argmax(lg))
    t0 = time.perf_counter()
    for _ in range(n_tok):
        tok = int(np.argmax(m.decode(st, tok)))
    dt = time.perf_counter() - t0
    log(f"cpu oracle: {n_tok} tokens in {dt:.1f}s")
    return {"value": round(n_tok / dt, 4), "unit": "tokens/s", "cores": cores,
            "kind": "oracle",
            "sample": f"AR greedy decode of {n_tok} tokens on the full {cfg['name']} "
                      f"model after a 32-token prompt (context ~{32 + n_tok}), fp32 "
                      f"numpy with {cores} BLAS threads; weights widened to fp32 "
                      f"before timing"}


if __name__ == "__main__":
    main()
