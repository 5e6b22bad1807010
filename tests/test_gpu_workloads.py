"""The measured workloads at full size on the GPU, checked against the
oracle on the outputs it can afford (the first generated tokens of a
request, a sample of the batched requests) and against the GPU's own
autoregressive run for the rest (spec decoding must emit the same tokens,
except at the GPU's own near-ties).

These tests generate multi-GB weights and run the CPU oracle on the full
models, so they take minutes; they print progress as they go.
"""

import gc
import time

import numpy as np
import pytest

import synth
from oracle.verify import argmax_lowest, top2_margin
from parity import NEAR_TIE, protocol_f, engine_for, oracle_for

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(1100)]

_W = {}


def _weights(name):
    if name not in _W:
        _W.clear()
        gc.collect()
        cfg = synth.model_config(name)
        t = time.time()
        _W[name] = (cfg, synth.make_weights(cfg))
        _say(f"[{name}] weights in {time.time() - t:.1f}s")
    return _W[name]


def _say(*a):
    print(*a, flush=True)


def _oracle_ref(orc, prompt, n, tag, chunk=512):
    """The oracle's greedy continuation (S, logits, margins) of n tokens,
    printing progress so a long CPU run is visibly alive."""
    t = time.time()
    st = orc.new_state()
    for s in range(0, len(prompt), chunk):
        lg = orc.append(st, prompt[s:s + chunk])[-1]
        _say(f"[{tag}] oracle prefill {min(s + chunk, len(prompt))}/{len(prompt)} "
             f"({time.time() - t:.0f}s)")
    S, L, M = [], [], []
    for i in range(n):
        L.append(lg)
        M.append(top2_margin(lg))
        S.append(argmax_lowest(lg))
        if i + 1 < n:
            lg = orc.decode(st, S[-1])
        if i % 4 == 3:
            _say(f"[{tag}] oracle token {i + 1}/{n} ({time.time() - t:.0f}s)")
    return np.array(S, np.int32), np.array(L, np.float32), np.array(M, np.float32)


_REF = {}


@pytest.mark.parametrize("fmt", ["w12", "native"])
def test_workload_dense8b_chain_full_size(fmt):
    """8B-shaped model, 2048-token prompt, chain K=16, alpha=0.7: the first
    32 generated tokens and their logits against the oracle, with the
    weights stored as W12 (as the benchmark runs it) and as bf16."""
    w = synth.workload("dense8b_chain")
    cfg, W = _weights(w["model"])
    eng = engine_for(cfg, W, max_ctx=w["prompt"] + 600, max_nodes=w["K"] + 1,
                     weight_format=fmt)
    prompt = synth.prompt_tokens(cfg["vocab"], w["prompt"], w["index"])
    orc = oracle_for(cfg, W, max_pos=4096)
    if "dense8b_chain" not in _REF:
        _REF["dense8b_chain"] = _oracle_ref(orc, prompt, 32, "8B chain")
    ref = _REF["dense8b_chain"]
    rep = protocol_f(eng, cfg, orc, prompt, 32, w, "chain", cfg_index=w["index"],
                     oracle_ref=ref)
    _say(rep)
    assert rep.first_bad is None and rep.max_logit_err <= 1.0, rep
    eng.close()


def test_workload_dense8b_tree_full_size():
    """8B-shaped model, 4096-token prompt, 64-node best-first trees
    (depth <= 8, alpha = 0.8 on the main path): 24 tokens against the
    oracle."""
    w = synth.workload("dense8b_tree")
    cfg, W = _weights(w["model"])
    eng = engine_for(cfg, W, max_ctx=w["prompt"] + 600, max_nodes=w["K"] + 1)
    prompt = synth.prompt_tokens(cfg["vocab"], w["prompt"], w["index"])
    orc = oracle_for(cfg, W, max_pos=8192)
    ref = _oracle_ref(orc, prompt, 24, "8B tree")
    rep = protocol_f(eng, cfg, orc, prompt, 24, w, "tree", cfg_index=w["index"],
                     oracle_ref=ref)
    _say(rep)
    assert rep.first_bad is None and rep.max_logit_err <= 1.0, rep
    eng.close()


def test_workload_dense8b_batched_full_size():
    """32 requests, contexts ~ U{512..4096} in 16-token pages, chain K=8 with
    per-request alpha ~ U(0.4, 0.9), one fused verify per step.  Every
    request must emit its own GPU-autoregressive continuation; the three
    shortest requests are also checked against the oracle."""
    w = synth.workload("dense8b_batched")
    cfg, W = _weights(w["model"])
    V, B, K, n_gen = cfg["vocab"], w["batch"], w["K"], 24
    ctx, alpha = synth.batched_mix(B, w["ctx_lo"], w["ctx_hi"], w["alpha_lo"],
                                   w["alpha_hi"])
    eng = engine_for(cfg, W, max_requests=B, max_ctx=int(ctx.max()) + 64,
                     max_nodes=K + 1, max_rows=B * (K + 1))
    prompts = [synth.prompt_tokens(V, int(ctx[r]), w["index"], r) for r in range(B)]
    t = time.time()
    firsts = [eng.prefill(r, prompts[r]) for r in range(B)]
    _say(f"[batched] prefill of {int(ctx.sum())} tokens in {time.time() - t:.1f}s")
    # GPU autoregressive reference for all requests at once (K = 0 rows)
    S_gpu = [[f] for f in firsts]
    marg = [[] for _ in range(B)]
    for step in range(n_gen - 1):
        paths, bonus, lg = eng.verify(list(range(B)), [[]] * B, [[]] * B, logits=True)
        lg = lg.cpu().numpy()
        for r in range(B):
            marg[r].append(top2_margin(lg[r]))
            S_gpu[r].append(bonus[r])
        eng.commit(list(range(B)), [[]] * B, bonus)
    for r in range(B):
        eng.release(r)
    # oracle check of the three shortest requests
    orc = oracle_for(cfg, W, max_pos=8192)
    for r in np.argsort(ctx)[:3]:
        S, L, M = _oracle_ref(orc, prompts[r], 12, f"batched req {r}")
        for t in range(12):
            if S_gpu[r][t] != S[t]:
                assert M[t] < NEAR_TIE, (r, t)
                break
    # spec decoding, one fused verify for all live requests per step
    for r in range(B):
        assert eng.prefill(r, prompts[r]) == S_gpu[r][0]
    g = [1] * B
    S_arr = [np.array(s, np.int32) for s in S_gpu]
    step, mism, rows = 0, 0, 0
    while min(g) < n_gen:
        live = [r for r in range(B) if g[r] < n_gen]
        dr = [synth.chain_drafts(S_arr[r], g[r], K, float(alpha[r]), V, w["index"], r, step)
              for r in live]
        paths, bonus = eng.verify(live, [d[0] for d in dr], [d[1] for d in dr])
        keep, roots = [], []
        for k, r in enumerate(live):
            em = [int(dr[k][0][p]) for p in paths[k]] + [bonus[k]]
            n_ok = 0
            for j, tk in enumerate(em):
                if g[r] + j >= n_gen or tk != S_gpu[r][g[r] + j]:
                    break
                n_ok += 1
            if n_ok < len(em) and g[r] + n_ok < n_gen:
                mism += 1
                assert marg[r][g[r] + n_ok - 1] < NEAR_TIE, (r, g[r] + n_ok)
                kp = paths[k][:n_ok] if n_ok < len(paths[k]) else paths[k]
                keep.append(kp)
                roots.append(S_gpu[r][g[r] + n_ok])
                g[r] += len(kp) + 1
            else:
                keep.append(paths[k])
                roots.append(bonus[k])
                g[r] += len(em)
        rows += sum(K + 1 for _ in live)
        eng.commit(live, keep, roots)
        step += 1
    _say(f"[batched] {step} fused steps, {rows} rows, GPU near-tie mismatches {mism}")
    eng.close()


def test_workload_hybrid27b_tree_full_size():
    """27B-shaped hybrid (48 recurrent + 16 attention layers), 2048-token
    prompt, 32-node trees that fork the recurrent state per branch: 12
    tokens against the oracle."""
    w = synth.workload("hybrid27b_tree")
    cfg, W = _weights(w["model"])
    eng = engine_for(cfg, W, max_ctx=w["prompt"] + 200, max_nodes=w["K"] + 1)
    prompt = synth.prompt_tokens(cfg["vocab"], w["prompt"], w["index"])
    orc = oracle_for(cfg, W, max_pos=4096)
    ref = _oracle_ref(orc, prompt, 12, "27B hybrid")
    rep = protocol_f(eng, cfg, orc, prompt, 12, w, "tree", cfg_index=w["index"],
                     oracle_ref=ref)
    _say(rep)
    assert rep.first_bad is None and rep.max_logit_err <= 1.0, rep
    eng.close()
