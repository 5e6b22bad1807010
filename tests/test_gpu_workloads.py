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
    (depth <= 8, alpha = 0.8 on the main path): 32 tokens against the
    oracle."""
    w = synth.workload("dense8b_tree")
    cfg, W = _weights(w["model"])
    eng = engine_for(cfg, W, max_ctx=w["prompt"] + 600, max_nodes=w["K"] + 1)
    prompt = synth.prompt_tokens(cfg["vocab"], w["prompt"], w["index"])
    orc = oracle_for(cfg, W, max_pos=8192)
    ref = _oracle_ref(orc, prompt, 32, "8B tree")
    rep = protocol_f(eng, cfg, orc, prompt, 32, w, "tree", cfg_index=w["index"],
                     oracle_ref=ref)
    _say(rep)
    assert rep.first_bad is None and rep.max_logit_err <= 1.0, rep
    eng.close()


def test_workload_dense8b_batched_full_size():
    """32 requests, contexts ~ U{512..4096} in 16-token pages, chain K=8 with
    per-request alpha ~ U(0.4, 0.9), one fused verify of up to 288 rows per
    step.  The three shortest requests follow the oracle: their drafts come
    from the oracle's greedy sequence, and every emitted token and the
    logits of every root and accepted row of the fused pass are compared
    with the oracle's.  Every other request must emit its own GPU
    autoregressive continuation (exact except at the GPU's own near-ties)."""
    w = synth.workload("dense8b_batched")
    cfg, W = _weights(w["model"])
    V, B, K, n_gen = cfg["vocab"], w["batch"], w["K"], 32
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
    # the oracle's greedy continuation of the three shortest requests
    orc = oracle_for(cfg, W, max_pos=8192)
    checked = [int(r) for r in np.argsort(ctx)[:3]]
    oref = {r: _oracle_ref(orc, prompts[r], n_gen, f"batched req {r}") for r in checked}
    # reference sequence per request: the oracle's for the checked ones
    ref = [np.array(oref[r][0] if r in oref else S_gpu[r], np.int32) for r in range(B)]
    for r in range(B):
        first = eng.prefill(r, prompts[r])
        if first != ref[r][0]:
            assert r in oref and oref[r][2][0] < NEAR_TIE, (r, first, ref[r][0])
            eng.force_root(r, int(ref[r][0]))
    # spec decoding, one fused verify for all live requests per step
    g = [1] * B
    step, mism, rows, ties, n_rows_checked, worst = 0, 0, 0, 0, 0, 0.0
    while min(g) < n_gen:
        live = [r for r in range(B) if g[r] < n_gen]
        dr = [synth.chain_drafts(ref[r], g[r], K, float(alpha[r]), V, w["index"], r, step)
              for r in live]
        paths, bonus, lg = eng.verify(live, [d[0] for d in dr], [d[1] for d in dr],
                                      logits=True)
        row0 = np.cumsum([0] + [len(d[0]) + 1 for d in dr])
        keep, roots = [], []
        for k, r in enumerate(live):
            em = [int(dr[k][0][p]) for p in paths[k]] + [bonus[k]]
            n_ok = 0
            for j, tk in enumerate(em):
                if g[r] + j >= n_gen or tk != ref[r][g[r] + j]:
                    break
                n_ok += 1
            if r in oref:
                # logits of the root and the accepted rows up to the first
                # mismatch, against the oracle's AR logits at those positions
                S, L, M = oref[r]
                idx = [0] + [p + 1 for p in paths[k]]
                n_cmp = min(len(idx), n_ok + 1, n_gen - g[r])
                got = lg[[int(row0[k]) + i for i in idx[:n_cmp]]].cpu().numpy()
                for i in range(n_cmp):
                    want = L[g[r] + i]
                    tol = 2e-2 * float(np.std(want))
                    worst = max(worst, float(np.max(np.abs(got[i] - want))) / tol)
                    n_rows_checked += 1
            if n_ok < len(em) and g[r] + n_ok < n_gen:
                if r in oref:
                    assert oref[r][2][g[r] + n_ok] < NEAR_TIE, (r, g[r] + n_ok)
                    ties += 1
                else:
                    assert marg[r][g[r] + n_ok - 1] < NEAR_TIE, (r, g[r] + n_ok)
                    mism += 1
                kp = paths[k][:n_ok] if n_ok < len(paths[k]) else paths[k]
                keep.append(kp)
                roots.append(int(ref[r][g[r] + n_ok]))
                g[r] += len(kp) + 1
            else:
                keep.append(paths[k])
                roots.append(bonus[k])
                g[r] += len(em)
        rows += sum(len(d[0]) + 1 for d in dr)
        eng.commit(live, keep, roots)
        step += 1
    _say(f"[batched] {step} fused steps, {rows} rows; oracle-checked requests "
         f"{checked}: {n_rows_checked} rows, max logit error {worst:.3f} x tolerance, "
         f"near-tie exemptions {ties}; GPU near-tie mismatches {mism}")
    assert worst <= 1.0
    eng.close()


def test_workload_hybrid27b_tree_full_size():
    """27B-shaped hybrid (48 recurrent + 16 attention layers), 2048-token
    prompt, 32-node trees that fork the recurrent state per branch: 32
    tokens against the oracle."""
    w = synth.workload("hybrid27b_tree")
    cfg, W = _weights(w["model"])
    eng = engine_for(cfg, W, max_ctx=w["prompt"] + 200, max_nodes=w["K"] + 1)
    prompt = synth.prompt_tokens(cfg["vocab"], w["prompt"], w["index"])
    orc = oracle_for(cfg, W, max_pos=4096)
    ref = _oracle_ref(orc, prompt, 32, "27B hybrid")
    rep = protocol_f(eng, cfg, orc, prompt, 32, w, "tree", cfg_index=w["index"],
                     oracle_ref=ref)
    _say(rep)
    assert rep.first_bad is None and rep.max_logit_err <= 1.0, rep
    eng.close()
