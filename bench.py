"""Benchmark of the speculative-decoding verify step on one MI355X.

Headline workload (the largest one-GPU configuration): the 27B-shaped
hybrid target (64 layers: 48 gated diagonal recurrent layers and 16 GQA
attention layers, d=5120, FFN 17408, vocab 151936, bf16 weights, random
init), 2048-token random prompt, batch 1, 32-node best-first draft trees
(depth <= 8, branching 4,3,2,2,1,1,1,1) whose main path copies the target's
own greedy continuation with match probability 0.8 per position.  Weights
are stored as W12 (lossless 12-bit tiles whose GEMM results are bitwise
those of bf16 storage) up to 40 rows per pass, bf16 above.  A step is one
spec_verify + spec_commit.

The other measured workloads are reported beside it (`other_workloads`):
the 8B-shaped dense decoder with chain drafts K=16 at a 2048-token prompt
(alpha 0.7, with 0.5 and 0.9), with 64-node trees at a 4096-token prompt,
and 32 batched requests (contexts 512..4096 in 16-token pages, chains of
K=8, alpha 0.4..0.9 per request) verified in one fused pass per step.
--workload NAME runs one workload alone as the headline.

Reported per workload: accepted tokens/s (emitted tokens over the summed
wall time of the verify + commit calls, inputs resident in HBM; host draft
synthesis excluded), the same at the closed-form expected tokens per step,
the device time of a step and its byte lower bound (max(FLOPs at 60% of 2.5
PFLOP/s, bytes at 90% of 8 TB/s), weights counted in their stored format)
and the fraction of it reached, the GPU autoregressive rate (K=0, same
library), and for the dominant kernel (the FFN gate/up GEMM) algorithmic
GB/s from per-launch HIP events against the 8 TB/s HBM peak.  Also: the
device's streaming-read ceiling measured live by the library's read probe,
and the CPU oracle's AR decode rate on a bounded sample of the headline
workload, as a reported baseline.
"""

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # MI355X HBM3E, bytes/s
PEAK_BF16 = 2.5e15         # MI355X dense bf16 MFMA, FLOP/s

WORKLOADS = ("dense8b_chain", "dense8b_tree", "dense8b_batched", "hybrid27b_tree")
HEADLINE = "hybrid27b_tree"
DEFAULT_STEPS = {"hybrid27b_tree": 200, "dense8b_chain": 100, "dense8b_tree": 80,
                 "dense8b_batched": 40}


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


def describe(name, w, alpha, planned, budget, choices, two):
    if name == "dense8b_batched":
        d = ("8B-shaped dense decoder, 32 requests (contexts 512..4096 in 16-token pages), "
             "chain drafts K=8, alpha 0.4..0.9 per request, one fused verify per step")
        if planned:
            d += (", draft lengths planned per step (8/12/16 by acceptance, shared budget of "
                  f"{budget} draft nodes)")
        return d
    if two:
        return ("8B-shaped dense decoder, 2048-token prompt, two-level verification: "
                f"{two[0]} drafts through the 8-bit weight view, candidate chain + {two[1]} "
                f"continuation drafts through the exact pass, alpha={alpha:.1f}, batch 1")
    if w["draft"] == "tree":
        model = ("8B-shaped dense decoder" if w["model"] == "dense8b" else
                 "27B-shaped hybrid (48 recurrent + 16 attention layers)")
        return (f"{model}, {w['prompt']}-token prompt, best-first draft tree of {w['K']} "
                f"nodes (depth <= {w['max_depth']}), alpha={alpha} on the main path, batch 1")
    return ("8B-shaped dense decoder, 2048-token prompt, chain draft K=16, "
            "alpha=%.1f, batch 1" % alpha)


def expected_tokens(w, alpha, alphas=None):
    """Closed-form expected tokens per step of the synthetic drafts: chains
    and the tree's main path accept each position independently with
    probability alpha (off-path tree nodes never match), so E = 1 +
    sum_{j<=depth} alpha^j; batched: the sum over requests."""
    import synth
    if w["name"] == "dense8b_batched":
        return float(sum(synth.expected_tokens_per_step(float(a), w["K"]) for a in alphas))
    depth = w.get("max_depth", 8) if w["draft"] == "tree" else w["K"]
    return synth.expected_tokens_per_step(alpha, depth)


def measure_workload(name, args, W_cache, steps, warmup, sweep=True):
    """Run one workload end to end on the GPU; returns a result dict (and
    the host weights, for the CPU baseline)."""
    import numpy as np
    import torch
    import synth
    from tree_verification_spec_amd import Engine, costmodel
    import tree_verification_spec_amd as L

    w = synth.workload(name)
    cfg = synth.model_config(w["model"])
    weights = args.weights
    if weights is None:
        rows = w["K"] + 1 if name != "dense8b_batched" else w["batch"] * (w["K"] + 1)
        weights = "w12" if rows <= 40 else "native"
    V, K, idx = cfg["vocab"], w["K"], w["index"]
    batched = name == "dense8b_batched"
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
    sweep_alphas = [] if (not sweep or args.no_sweep or batched or tree) else \
        [a for a in w.get("alphas", ()) if abs(a - alpha_main) > 1e-9]
    planned = batched and args.policy == "budget"
    two = tuple(int(x) for x in args.two_level.split(",")) if args.two_level else None
    if two and (batched or tree):
        print("bench.py: --two-level is for the chain workload", file=sys.stderr)
        sys.exit(2)
    if two:
        weights = "w12_lowp"
    choices, min_prob, decay = (8, 12, 16), 0.05, 0.9
    budget = B * K
    depth = w.get("max_depth", 8) if tree else (max(choices) if planned else K)
    if two:
        depth = two[0] + two[1] + 1
    n_timing = max(10, steps // 4)
    runs = [(alpha_main if not batched else 0.9, warmup + steps),
            (alpha_main if not batched else 0.9, n_timing + 2)]
    runs += [(a, max(20, steps // 2) + 4) for a in sweep_alphas]
    need = max(synth.expected_tokens_per_step(a, depth) * n for a, n in runs)
    ref_len = args.ref_len or min(int(need * 1.5) + 64, (depth + 1) *
                                  max(n for _, n in runs) + 8)

    if W_cache.get("model") != w["model"]:
        W_cache.clear()
        gc.collect()
        t0 = time.time()
        W_cache["W"] = synth.make_weights(cfg)
        W_cache["model"] = w["model"]
        log(f"[{name}] weights generated in {time.time() - t0:.1f}s")
    W = W_cache["W"]
    max_ctx = (max(len(p) for p in prompts) + 2 * (depth + 1) +
               max(ref_len, (depth + 1) * max(n for _, n in runs)))
    eng = Engine(cfg, device=0, max_requests=B, max_ctx=max_ctx,
                 max_nodes=(max(choices) if planned else K) + 1,
                 max_rows=B * ((depth if two else K) + 1), prefill_chunk=512,
                 weight_format=weights)
    t0 = time.time()
    eng.load_weights([W[n] for n, _, _ in synth.tensor_specs(cfg)])
    log(f"[{name}] weights loaded in {time.time() - t0:.1f}s")

    # ---- GPU autoregressive reference (K = 0): continuations + AR rate
    sync = torch.cuda.synchronize
    t0 = time.time()
    S = [[eng.prefill(r, prompts[r])] for r in range(B)]
    sync()
    log(f"[{name}] prefill of {sum(len(p) for p in prompts)} tokens in {time.time() - t0:.1f}s")
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
    log(f"[{name}] GPU AR: {ref_len - 1} tokens x {B} requests, {ar_tps:.1f} tok/s")

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
                nb, fl, lb, ty = step_bounds(cfg, [k + 1 for k in lens], ctx, weights)
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

    res = run(alpha_main, steps, warmup)
    log(f"[{name}] alpha={alpha_main}: {res}")
    # the dominant kernel's launch times: each gate/up launch records its own
    # start and end in a HIP event pair (extended launch; passes of this run
    # are launched kernel by kernel, without graph replay)
    rl = run(alpha_main, n_timing, 2, timing_cls=1)
    log(f"[{name}] timed launches: {rl}")
    sweep_out = {}
    for al in sweep_alphas:
        r = run(al, max(20, steps // 2), 4)
        sweep_out[str(al)] = dict(tokens_per_s=round(r["tps"], 1),
                                  tokens_per_step=round(r["tok_per_step"], 3),
                                  lb_frac=round(r["lb_ms"] / r["dev_ms"], 4))
        log(f"[{name}] alpha={al}: {r}")
    if sweep_alphas:
        sweep_out[str(alpha_main)] = dict(tokens_per_s=round(res["tps"], 1),
                                          tokens_per_step=round(res["tok_per_step"], 3),
                                          lb_frac=round(res["lb_ms"] / res["dev_ms"], 4))
    eng.close()
    del eng
    gc.collect()
    torch.cuda.empty_cache()

    # roofline of the dominant kernel: FFN gate/up GEMM, weights streamed once
    # per launch (passes of more than 128 rows launch it once per 128 rows;
    # the bytes still count the weights once)
    gu_bytes = costmodel.weight_bytes(2 * cfg["ffn_dim"], cfg["d_model"], weights)
    k_ms, k_n = rl["ktime"]
    k_avg_s = k_ms / 1e3 / max(1, k_n)
    achieved = gu_bytes / k_avg_s / 1e9
    e_tok = expected_tokens(w, alpha_main, alphas)
    out = {
        "workload": describe(name, w, alpha_main, planned, budget, choices, two),
        "name": name, "batch": B, "draft_K": K, "alpha": alpha_main,
        "prompt": None if batched else w["prompt"], "weights": weights,
        "policy": (f"budget {budget}, lengths {list(choices)}, min_prob {min_prob}, "
                   f"decay {decay}") if planned else "fixed",
        "steps": steps, "warmup": warmup,
        "tokens_per_s": round(res["tps"], 2),
        "ms_per_step": round(res["ms"], 4),
        "tokens_per_step": round(res["tok_per_step"], 3),
        "expected_tokens_per_step": round(e_tok, 3),
        "tokens_per_s_at_expected": round(e_tok / (res["ms"] / 1e3), 2),
        "verify_step": {
            "device_ms_median": round(res["dev_ms"], 4),
            "byte_lower_bound_ms": round(res["lb_ms"], 4),
            "lb_frac": round(res["lb_ms"] / res["dev_ms"], 4),
            "algorithmic_GBps": round(res["bytes"] / (res["dev_ms"] / 1e3) / 1e9, 1),
            "device_ms_p10_p50_p90": [round(x, 4) for x in res["dev_pct"]],
            "forced_mismatches": res["mism"],
        },
        "ar_tokens_per_s": round(ar_tps, 2),
        "speedup_over_ar": round(res["tps"] / ar_tps, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM / 1e9, "unit": "GB/s",
                     "frac": round(achieved / (PEAK_HBM / 1e9), 4),
                     "traffic": measured_traffic(name, weights),
                     "kernel": "FFN gate/up GEMM + SwiGLU (%.1f MB of %s weights per launch)"
                               % (gu_bytes / 1e6, "W12" if weights == "w12" else "bf16"),
                     "launches": k_n, "avg_launch_us": round(k_avg_s * 1e6, 2)},
        "cost_model": {
            "rows": B * (K + 1),
            "types": {t: {"bytes": b, "flops": f,
                          "bound_us": round(1e6 * costmodel.lower_bound(b, f), 2)}
                      for t, (b, f) in res["types"].items()},
        },
    }
    if sweep_out:
        out["alpha_sweep"] = sweep_out
    return out, cfg, W


def stream_ceiling(kernel_bytes):
    """The device's streaming-read bandwidth from the library's read probe
    (the weight GEMMs' access pattern: 1 KB blocks per wavefront, loads in
    flight, all wavefronts sweeping the buffer together), MALL-cold: each
    launch reads a region not read by the previous ones.  Best of a few
    launch shapes per size: the dominant kernel's weight bytes, and 1 GiB."""
    import torch
    import tree_verification_spec_amd as L
    GiB, MiB = 1 << 30, 1 << 20
    buf = torch.empty(2 * GiB, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.empty(1 << 16, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream()
    out = {}
    shapes = [(256, 8, 4), (256, 8, 8), (192, 4, 8), (512, 8, 4)]
    for size in (int(kernel_bytes), 1024 * MiB):
        best = None
        for grid, waves, depth in shapes:
            tw = grid * waves
            sz = size // (1024 * tw) * (1024 * tw)
            nreg = (2 * GiB) // sz
            times = []
            for r in range(6):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(st)
                L.spec_probe_read_bandwidth(buf.data_ptr() + (r % nreg) * sz, sz, grid, waves,
                                            depth, 1, sink.data_ptr(), st.cuda_stream)
                e1.record(st)
                e1.synchronize()
                if r >= 2:
                    times.append(e0.elapsed_time(e1))
            gbps = sz / (sorted(times)[len(times) // 2] / 1e3) / 1e9
            if best is None or gbps > best[0]:
                best = (gbps, grid, waves, depth)
        out[f"{size / MiB:.1f}MiB"] = {"GBps": round(best[0], 1), "grid": best[1],
                                       "waves": best[2], "depth": best[3]}
    del buf, sink
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps of the headline workload (default: 200 for the 27B "
                         "hybrid; the other workloads use their own defaults)")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default=None, choices=WORKLOADS,
                    help="run only this workload, as the headline")
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
    ap.add_argument("--no-others", action="store_true",
                    help="skip the other workloads (headline only)")
    ap.add_argument("--no-stream", action="store_true", help="skip the read-ceiling probe")
    ap.add_argument("--cpu-tokens", type=int, default=16)
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

    import torch
    import tree_verification_spec_amd as L
    L.lib()

    if args.copy_probe_bytes:
        n = args.copy_probe_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)        # an elementwise kernel: reads n*4, writes n*4
        torch.cuda.synchronize()
        del src, dst
        log(f"copy probe: {4 * n} bytes")

    headline = args.workload or HEADLINE
    others = [] if (args.workload or args.no_others) else \
        [w for w in WORKLOADS if w != headline]
    W_cache = {}
    other_out = {}
    # the 8B workloads first (they share one set of host weights), then the
    # headline (its host weights stay for the CPU baseline)
    for name in others:
        r, _, _ = measure_workload(name, args, W_cache, DEFAULT_STEPS[name], 4)
        other_out[name] = r
    steps = args.steps if args.steps is not None else DEFAULT_STEPS[headline]
    head, cfg, W = measure_workload(headline, args, W_cache, steps, args.warmup)
    from tree_verification_spec_amd import costmodel
    ceiling = None if args.no_stream else stream_ceiling(
        costmodel.weight_bytes(2 * cfg["ffn_dim"], cfg["d_model"], head["weights"]))
    if ceiling:
        log(f"stream read ceiling: {ceiling}")
        first = next(iter(ceiling.values()))
        head["roofline"]["frac_of_read_ceiling"] = round(
            head["roofline"]["achieved"] / first["GBps"], 4)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, W, args.cpu_tokens)

    out = {
        "metric": "accepted tokens/s at batch 1 + verify-step HBM GB/s vs byte lower bound",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (random-init weights N(0,0.02), uniform random prompt, "
                "drafts from the target's greedy continuation)",
        "config": {k: head[k] for k in ("workload", "name", "batch", "draft_K", "alpha",
                                       "prompt", "weights", "policy")},
        "tokens_per_step": head["tokens_per_step"],
        "expected_tokens_per_step": head["expected_tokens_per_step"],
        "tokens_per_s_at_expected": head["tokens_per_s_at_expected"],
        "verify_step": head["verify_step"],
        "ar_tokens_per_s": head["ar_tokens_per_s"],
        "speedup_over_ar": head["speedup_over_ar"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "stream_read_ceiling": ceiling,
        "cost_model": head["cost_model"],
        "other_workloads": other_out,
    }
    if "alpha_sweep" in head:
        out["alpha_sweep"] = head["alpha_sweep"]
    print(json.dumps(out), flush=True)


def traffic_file(name, fmt):
    tag = {"w12": "w12", "native": "bf16"}.get(fmt)
    if tag is None:
        return None
    return os.path.join(ROOT, "profiles", f"gemm_gateup_swiglu_{tag}_{name}_traffic.md")


def measured_traffic(name, fmt):
    """HBM bytes per gate/up launch from the committed counter summary for
    this workload and weight format (FETCH_SIZE + WRITE_SIZE, scaled by a
    plain copy of known size), or None when there is none or the kernel
    sources changed since the counters were taken."""
    from tree_verification_spec_amd import counters
    try:
        kv = counters.read_summary_fields(traffic_file(name, fmt))
        if kv.get("kernel_source_sha256_16") != counters.kernel_source_hash():
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, TypeError, KeyError, ValueError):
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
