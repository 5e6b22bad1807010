"""GPU parity: the HIP verify path (through the C ABI) against the oracle.

Tokens must equal the oracle's greedy output except where the oracle's
top-1/top-2 margin is below 1e-2 (counted); logits must be within 1e-4
(fp32 models) or 2e-2 x the row's logit std (bf16 models).
"""

import numpy as np
import pytest

import synth
from oracle import ar_greedy, top2_margin
from parity import (NEAR_TIE, protocol_f, engine_for, oracle_for, make_drafts,
                    logit_tol)

pytestmark = pytest.mark.gpu

_CACHE = {}


def _setup(name):
    if name not in _CACHE:
        cfg = synth.model_config(name)
        _CACHE[name] = (cfg, synth.make_weights(cfg))
    return _CACHE[name]


def _say(*a):
    print(*a, flush=True)


def _assert_ok(rep, max_tie_frac=0.2):
    _say(rep)
    assert rep.first_bad is None, rep
    assert rep.max_logit_err <= 1.0, rep
    assert rep.near_tie_mismatch <= max(1, int(max_tie_frac * rep.emitted)), rep


# --------------------------------------------------------------- workload 0

def test_tiny_chain_workload():
    """Tiny fp32 decoder, 64-token prompt, chain K=4, alpha=0.7, 128 tokens;
    every row's logits (rejected drafts included) against the oracle's
    tree-masked pass."""
    w = synth.workload("tiny_chain")
    cfg, W = _setup("tiny")
    eng = engine_for(cfg, W, max_ctx=512, max_nodes=w["K"] + 1)
    orc = oracle_for(cfg, W)
    prompt = synth.prompt_tokens(cfg["vocab"], w["prompt"], w["index"])
    rep = protocol_f(eng, cfg, orc, prompt, w["gen"], w, "chain",
                     cfg_index=w["index"], all_rows=True)
    _assert_ok(rep)
    e = synth.expected_tokens_per_step(w["alpha"], w["K"])
    _say("tokens/step", rep.emitted / rep.steps, "expected", e)


@pytest.mark.parametrize("name", ["tiny_gqa", "tiny_hybrid", "tiny_gqa_bf16",
                                  "tiny_hybrid_bf16"])
@pytest.mark.parametrize("kind", ["chain", "tree"])
def test_small_models(name, kind):
    cfg, W = _setup(name)
    w = dict(K=8 if kind == "chain" else 20, alpha=0.8,
             branching=(4, 3, 2, 2, 1, 1, 1, 1), max_depth=8)
    eng = engine_for(cfg, W, max_ctx=512, max_nodes=w["K"] + 1)
    orc = oracle_for(cfg, W)
    prompt = synth.prompt_tokens(cfg["vocab"], 37, 50)
    rep = protocol_f(eng, cfg, orc, prompt, 40, w, kind, cfg_index=50,
                     all_rows=True)
    _assert_ok(rep)


@pytest.mark.parametrize("name", ["tiny", "tiny_gqa", "tiny_gqa_bf16", "tiny_hybrid_bf16"])
@pytest.mark.parametrize("kind", ["chain", "tree", "bigtree"])
def test_streamed_attention_small_models(name, kind):
    """Attention streamed in stages of 64 keys in two key ranges per
    request, KV head and query group (the debug flag), so a range spans
    several stages and ends in a partial one, on chains and trees whose
    query tiles per KV head leave 4, 2 or 1 key blocks in flight per tile
    (tiny: one tile per chain pass; the GQA models: 3 tiles per chain pass,
    6 per tree pass, and 41-node trees of 11 tiles in two query groups);
    every row's logits against the oracle's tree-masked pass."""
    cfg, W = _setup(name)
    K = {"chain": 4 if name == "tiny" else 8, "tree": 20, "bigtree": 40}[kind]
    w = dict(K=K, alpha=0.8, branching=(6, 4, 3, 2, 2, 1, 1, 1), max_depth=8)
    kind = "chain" if kind == "chain" else "tree"
    eng = engine_for(cfg, W, max_ctx=512, max_nodes=w["K"] + 1)
    eng.debug_flags(2)
    orc = oracle_for(cfg, W)
    prompt = synth.prompt_tokens(cfg["vocab"], 301, 52)
    rep = protocol_f(eng, cfg, orc, prompt, 24, w, kind, cfg_index=52, all_rows=True)
    _assert_ok(rep)


def test_prefill_chunking_and_long_prompt():
    """A prompt spanning several prefill chunks and KV pages."""
    cfg, W = _setup("tiny_hybrid_bf16")
    w = dict(K=6, alpha=0.7)
    eng = engine_for(cfg, W, max_ctx=1024, max_nodes=7, prefill_chunk=96)
    orc = oracle_for(cfg, W)
    prompt = synth.prompt_tokens(cfg["vocab"], 333, 51)
    rep = protocol_f(eng, cfg, orc, prompt, 24, w, "chain", cfg_index=51,
                     all_rows=True)
    _assert_ok(rep)


# ---------------------------------------------------------------- batched

@pytest.mark.parametrize("planned,table_only,stream,pool", [
    (False, False, None, 0), (True, False, None, 0), (False, True, None, 0),
    (False, False, True, 0), (False, True, True, 0), (False, False, False, 0),
    (False, False, None, 40), (False, False, True, 40)])
def test_batched_requests(planned, table_only, stream, pool):
    """Several requests of different lengths in one fused verify per step,
    each checked against its own oracle greedy run (table_only: with every
    KV page looked up in the block table; stream: attention streamed in key
    ranges of several stages (True), or one key split staged per workgroup
    (False), forced by the debug flags; None: the planner's choice; pool: a
    KV pool of that many pages shared by the requests, which take pages as
    they grow, so a request's pages interleave with the others' (0: room for
    every request at max_ctx)).
    planned: each step's
    draft lengths come from the batch planner (lengths up to 2, 4 or 8 from
    the requests' acceptance so far, 16 draft nodes shared by 5 requests, so
    a request may offer none); the emitted tokens must not depend on it."""
    from tree_verification_spec_amd import spec_acceptance_update, spec_plan_drafts
    cfg, W = _setup("tiny_gqa_bf16")
    V = cfg["vocab"]
    n_req, K, n_gen = 5, 8, 30
    succ, fail = [0.0] * n_req, [0.0] * n_req
    lens_used = set()
    eng = engine_for(cfg, W, max_requests=8, max_ctx=512, max_nodes=K + 1,
                     max_rows=8 * (K + 1), kv_pages=pool)
    flags = (1 if table_only else 0) | {None: 0, True: 2, False: 4}[stream]
    if flags:  # every KV page through the block table; streamed or split attention
        eng.debug_flags(flags)
    orc = oracle_for(cfg, W)
    lens = [17, 40, 63, 100, 129]
    alphas = [0.4, 0.6, 0.7, 0.8, 0.9]
    reqs = [0, 3, 1, 7, 2]              # request ids need not be dense
    refs, g = [], []
    for i, r in enumerate(reqs):
        prompt = synth.prompt_tokens(V, lens[i], 60, i)
        S, L, M, _ = ar_greedy(orc, prompt, n_gen)
        refs.append((S, L, M))
        first = eng.prefill(r, prompt)
        if first != S[0]:
            assert M[0] < NEAR_TIE
            eng.force_root(r, int(S[0]))
        g.append(1)
    step, ties = 0, 0
    while min(g) < n_gen:
        live = [i for i in range(n_req) if g[i] < n_gen]
        if planned:
            plan = spec_plan_drafts([succ[i] for i in live], [fail[i] for i in live],
                                    [2, 4, 8], 0.05, 16)
            assert sum(plan) <= 16
            lens_used.update(plan)
        else:
            plan = [K] * len(live)
        drafts, parents = [], []
        for k, i in enumerate(live):
            t, p = synth.chain_drafts(refs[i][0], g[i], plan[k], alphas[i], V, 60, i, step)
            drafts.append(t)
            parents.append(p)
        paths, bonus, lg = eng.verify([reqs[i] for i in live], drafts, parents,
                                      logits=True)
        lg = lg.cpu().numpy()
        row0 = 0
        keep_all, roots = [], []
        for k, i in enumerate(live):
            S, L, M = refs[i]
            emitted = [int(drafts[k][p]) for p in paths[k]] + [bonus[k]]
            n_ok = 0
            for j, t in enumerate(emitted):
                if g[i] + j >= n_gen or t != S[g[i] + j]:
                    break
                n_ok += 1
            # logits of the root row and accepted rows before any mismatch
            rows = [row0] + [row0 + p + 1 for p in paths[k]]
            for j in range(min(n_ok + 1, len(rows))):
                if g[i] + j < n_gen:
                    tol = logit_tol(cfg["dtype"], L[g[i] + j])
                    assert np.max(np.abs(lg[rows[j]] - L[g[i] + j])) <= tol
            if n_ok < len(emitted) and g[i] + n_ok < n_gen:
                pos = g[i] + n_ok
                assert M[pos] < NEAR_TIE, (i, pos, emitted, S[g[i]:g[i] + 10])
                ties += 1
                keep = paths[k][:n_ok] if n_ok < len(paths[k]) else paths[k]
                keep_all.append(keep)
                roots.append(int(S[pos]))
                g[i] += len(keep) + 1
            else:
                keep_all.append(paths[k])
                roots.append(bonus[k])
                g[i] += len(emitted)
            row0 += len(drafts[k]) + 1
        eng.commit([reqs[i] for i in live], keep_all, roots)
        if planned:
            su, fa = spec_acceptance_update([len(d) for d in drafts],
                                            [len(p) for p in paths], 0.9,
                                            [succ[i] for i in live], [fail[i] for i in live])
            for k, i in enumerate(live):
                succ[i], fail[i] = su[k], fa[k]
        step += 1
    _say("batched steps", step, "near-tie mismatches", ties,
         "planned lengths", sorted(lens_used))
    assert ties <= 3
    if planned:
        assert len(lens_used) > 2 and max(lens_used) > 4


# ------------------------------------------------- spec == GPU AR (protocol A)

def test_kv_pool_exhaustion_and_reuse():
    """A pool of 6 KV pages for two requests: each prompt takes its pages at
    prefill; a verify that needs a page the pool no longer has fails with
    SPEC_E_CAPACITY and leaves the request as it was; after the other
    request is released, the same verify succeeds on a page that request
    held (so the request's pages are no longer consecutive, and attention
    reads them through the block table) and every row's logits match the
    oracle's."""
    from tree_verification_spec_amd._lib import SPEC_E_CAPACITY, SpecError
    cfg, W = _setup("tiny_gqa_bf16")
    V = cfg["vocab"]
    eng = engine_for(cfg, W, max_requests=2, max_ctx=256, max_nodes=5, kv_pages=6)
    orc = oracle_for(cfg, W)
    p0 = synth.prompt_tokens(V, 44, 61, 0)
    p1 = synth.prompt_tokens(V, 40, 61, 1)
    S, L, M, _ = ar_greedy(orc, p0, 6)
    eng.prefill(1, p1)                   # 40 tokens: pages 0-2
    first = eng.prefill(0, p0)           # 44 tokens: pages 3-5, the pool is empty
    root = first if first == S[0] else int(S[0])
    if first != S[0]:
        assert M[0] < NEAR_TIE
        eng.force_root(0, root)
    drafts = [np.array(S[1:5], np.int32)]  # positions 44..48: a fourth page
    parents = [np.arange(-1, 3, dtype=np.int32)]
    with pytest.raises(SpecError) as e:
        eng.verify([0], drafts, parents)
    assert e.value.code == SPEC_E_CAPACITY
    assert eng.state(0) == (44, root)
    eng.release(1)                       # request 0 then takes page 0 after 3-5
    paths, bonus, lg = eng.verify([0], drafts, parents, logits=True)
    lg = lg.cpu().numpy()
    # row j holds S[j] (the root, then the drafts): its logits are L[j + 1]
    for j in range(5):
        assert np.max(np.abs(lg[j] - L[j + 1])) <= logit_tol(cfg["dtype"], L[j + 1])
    if min(M[1:6]) >= NEAR_TIE:
        assert list(paths[0]) == [0, 1, 2, 3] and bonus[0] == S[5]
    eng.close()


def test_spec_equals_gpu_autoregressive():
    cfg, W = _setup("tiny")
    V, n_gen = cfg["vocab"], 60
    prompt = synth.prompt_tokens(V, 64, 0)
    eng = engine_for(cfg, W, max_ctx=512, max_nodes=5)
    # GPU AR: K = 0 verify steps
    S_gpu, marg = [eng.prefill(0, prompt)], []
    for t in range(n_gen - 1):
        paths, bonus, lg = eng.verify([0], [[]], [[]], logits=True)
        marg.append(top2_margin(lg[0].cpu().numpy()))
        eng.commit([0], [[]], [bonus[0]])
        S_gpu.append(bonus[0])
    eng.release(0)
    orc = oracle_for(cfg, W)
    S, _, M, _ = ar_greedy(orc, prompt, n_gen)
    for t in range(n_gen):
        if S_gpu[t] != S[t]:
            assert M[t] < NEAR_TIE
            break
    # spec decoding with drafts from the GPU's own AR sequence
    w = dict(K=4, alpha=0.7)
    first = eng.prefill(0, prompt)
    assert first == S_gpu[0]
    g, step, mism = 1, 0, 0
    while g < n_gen:
        toks, par = synth.chain_drafts(np.array(S_gpu), g, 4, 0.7, V, 0, 0, step)
        paths, bonus = eng.verify([0], [toks], [par])
        emitted = [int(toks[p]) for p in paths[0]] + [bonus[0]]
        n_ok = 0
        for j, t in enumerate(emitted):
            if g + j >= n_gen or t != S_gpu[g + j]:
                break
            n_ok += 1
        if n_ok < len(emitted) and g + n_ok < n_gen:
            mism += 1
            assert marg[g + n_ok - 1] < NEAR_TIE
            keep = paths[0][:n_ok] if n_ok < len(paths[0]) else paths[0]
            eng.commit([0], [keep], [S_gpu[g + n_ok]])
            g += len(keep) + 1
        else:
            eng.commit([0], paths, bonus)
            g += len(emitted)
        step += 1
    _say("spec vs GPU AR mismatches:", mism)


# ---------------------------------------------------------- fault injection

def test_fault_injection_is_caught_at_first_affected_token():
    """A logit bias switched on at a late position must make the checker
    fail exactly at the first generated token it affects."""
    w = synth.workload("tiny_chain")
    cfg, W = _setup("tiny")
    eng = engine_for(cfg, W, max_ctx=512, max_nodes=5)
    orc = oracle_for(cfg, W)
    prompt = synth.prompt_tokens(cfg["vocab"], 64, 0)
    S, L, M, _ = ar_greedy(orc, prompt, 96)
    after = 64 + 70        # positions >= after are biased
    t_star = after - 64 + 1
    bad_tok = int((S[t_star] + 1) % cfg["vocab"])
    eng.set_fault(bad_tok, 50.0, after)
    rep = protocol_f(eng, cfg, orc, prompt, 96, w, "chain", cfg_index=0,
                     oracle_ref=(S, L, M), check_logits=False)
    _say(rep)
    assert rep.first_bad is not None and rep.first_bad[0] == t_star
    assert rep.first_bad[1] == bad_tok


# -------------------------------------------------------------- error paths

def test_error_paths_leave_state_unchanged():
    from tree_verification_spec_amd import (SpecError, SPEC_E_INVAL,
                                            SPEC_E_STATE, SPEC_E_CAPACITY)
    cfg, W = _setup("tiny")
    V = cfg["vocab"]
    eng = engine_for(cfg, W, max_requests=2, max_ctx=96, max_nodes=5)
    prompt = synth.prompt_tokens(V, 64, 0)
    first = eng.prefill(0, prompt)
    state0 = eng.state(0)

    def code(f, *a):
        with pytest.raises(SpecError) as ei:
            f(*a)
        return ei.value.code
    assert code(eng.verify, [0], [[1, 2]], [[-1, 1]]) == SPEC_E_INVAL   # parent >= i
    assert code(eng.verify, [0], [[1, 2]], [[-2, 0]]) == SPEC_E_INVAL
    assert code(eng.verify, [0], [[V, 2]], [[-1, 0]]) == SPEC_E_INVAL   # token
    assert code(eng.verify, [0], [[1] * 5], [[-1, 0, 1, 2, 3]]) == SPEC_E_INVAL  # K+1 > max_nodes
    assert code(eng.verify, [1], [[1]], [[-1]]) == SPEC_E_STATE        # inactive
    assert code(eng.verify, [2], [[1]], [[-1]]) == SPEC_E_INVAL        # no such id
    assert code(eng.verify, [0, 0], [[1], [1]], [[-1], [-1]]) == SPEC_E_INVAL
    assert code(eng.commit, [0], [[]], [1]) == SPEC_E_STATE            # no verify
    assert eng.state(0) == state0
    paths, bonus = eng.verify([0], [[5, 6, 7]], [[-1, -1, 0]])
    assert code(eng.commit, [0], [[1, 2]], [1]) == SPEC_E_STATE         # not a root path
    assert code(eng.commit, [0], [[2]], [1]) == SPEC_E_STATE            # 2's parent is 0
    assert eng.state(0) == state0
    eng.commit([0], [[0]], [bonus[0]])                                  # any root path
    assert eng.state(0) == (state0[0] + 2, bonus[0])
    # capacity: 64 + 2 committed, max_ctx 96
    while True:
        n, _ = eng.state(0)
        if n + 5 > 96:
            break
        p, b = eng.verify([0], [[1, 2, 3, 4]], [[-1, 0, 1, 2]])
        eng.commit([0], [[]], b)
    st = eng.state(0)
    assert code(eng.verify, [0], [[1, 2, 3, 4]], [[-1, 0, 1, 2]]) == SPEC_E_CAPACITY
    assert eng.state(0) == st
    assert code(eng.prefill, 0, prompt) == SPEC_E_STATE                # active
    eng.release(0)
    assert code(eng.prefill, 0, list(range(95))) == SPEC_E_CAPACITY    # too long


def test_verify_is_deterministic():
    cfg, W = _setup("tiny_hybrid_bf16")
    eng = engine_for(cfg, W, max_ctx=512, max_nodes=17)
    prompt = synth.prompt_tokens(cfg["vocab"], 50, 52)
    eng.prefill(0, prompt)
    toks = np.arange(16) * 7 % cfg["vocab"]
    par = np.array([-1, 0, 0, 1, 2, 3, -1, 6, 7, 4, 9, 5, 11, 12, 8, 14])
    a = eng.verify([0], [toks], [par], logits=True)
    la = a[2].cpu().numpy()  # the logits view is reused by the next verify
    b = eng.verify([0], [toks], [par], logits=True)
    assert a[0] == b[0] and a[1] == b[1]
    assert np.array_equal(la, b[2].cpu().numpy())


def test_graph_replay_equals_individual_launches():
    """Verify passes replayed from captured graphs (the default) give the
    same paths, bonus tokens and logits as individually launched kernels:
    several replays of each captured pass (chain, tree, with and without
    logits), with eager commits and host synchronisation between them."""
    cfg, W = _setup("tiny_hybrid_bf16")
    V = cfg["vocab"]
    prompt = synth.prompt_tokens(V, 70, 54)
    rng = np.random.default_rng(54)
    tree_par = np.array([-1, 0, 0, 1, 2, 3, -1, 6, 7, 4, 9, 5])
    steps = []
    for k in range(12):
        if k % 2:
            steps.append((rng.integers(0, V, 12), tree_par, k % 4 == 1))
        else:
            steps.append((rng.integers(0, V, 8), np.arange(-1, 7), k % 4 == 0))
    runs = []
    for graphs in (True, False):
        eng = engine_for(cfg, W, max_ctx=512, max_nodes=17)
        eng.use_graphs(graphs)
        eng.prefill(0, prompt)
        out = []
        for toks, par, want_logits in steps:
            r = eng.verify([0], [toks], [par], logits=want_logits)
            lg = r[2].cpu().numpy().copy() if want_logits else None
            out.append((r[0], r[1], lg))
            eng.commit([0], r[0], r[1])
        runs.append(out)
        eng.close()
    for (pa, ba, la), (pb, bb, lb) in zip(*runs):
        assert pa == pb and ba == bb
        if la is not None:
            assert np.array_equal(la, lb)


def test_kernel_timing_counts_launches_and_leaves_results_unchanged():
    """Timed passes (each launch of one kernel class records its own start
    and end in a HIP event pair) give the same paths, bonus tokens and
    logits as untimed ones, one timed launch per layer (per pass for the LM
    head), and positive durations."""
    cfg, W = _setup("tiny_gqa_bf16")
    V = cfg["vocab"]
    prompt = synth.prompt_tokens(V, 40, 56)
    toks = np.arange(16) * 5 % V
    par = np.arange(-1, 15)
    eng = engine_for(cfg, W, max_ctx=512, max_nodes=17)
    eng.prefill(0, prompt)
    ref = eng.verify([0], [toks], [par], logits=True)
    ref_lg = ref[2].cpu().numpy().copy()
    n_layers = cfg["n_layers"]
    for cls, per_pass in ((1, n_layers), (2, n_layers), (3, 1), (4, n_layers)):
        eng.timing(cls)
        eng.timing_read()
        for _ in range(2):
            r = eng.verify([0], [toks], [par], logits=True)
            assert r[0] == ref[0] and r[1] == ref[1]
            assert np.array_equal(r[2].cpu().numpy(), ref_lg)
        ms, n = eng.timing_read()
        eng.timing(0)
        _say(f"timing class {cls}: {n} launches, {ms:.4f} ms")
        assert n == 2 * per_pass and 0.0 < ms < 1e3
    eng.close()


# ------------------------------------------------ full-width model variants

@pytest.mark.parametrize("name,budget", [("dense8b_l2", 64), ("hybrid27b_l4", 32)])
def test_full_width_trees(name, budget):
    """Real hidden size, heads, FFN and vocabulary with few layers; draft
    trees of the workloads' node budgets; every row's logits checked."""
    cfg, W = _setup(name)
    w = dict(K=budget, alpha=0.8, branching=(4, 3, 2, 2, 1, 1, 1, 1), max_depth=8)
    eng = engine_for(cfg, W, max_ctx=1024, max_nodes=budget + 1)
    orc = oracle_for(cfg, W)
    prompt = synth.prompt_tokens(cfg["vocab"], 300, 53)
    rep = protocol_f(eng, cfg, orc, prompt, 14, w, "tree", cfg_index=53,
                     all_rows=True)
    _assert_ok(rep)


# ------------------------------------------------ row-count invariance

def _main_path_tree(K, main_len, rng):
    """Parents of K draft nodes laid out like a best-first tree: the main
    path (a chain from the root) is interleaved in index order with other
    nodes hung off random earlier nodes, each main node being the first
    child of its parent (so the main path is the depth-first walk's first
    branch, not the lowest indices)."""
    par, main = [], []
    per = (K - main_len) // main_len
    for d in range(main_len):
        main.append(len(par))
        par.append(main[-2] if d else -1)
        for _ in range(per if d < main_len - 1 else K - len(par)):
            if len(par) >= K:
                break
            cand = [-1] + [i for i in range(len(par)) if i != main[-1]]
            par.append(int(rng.choice(cand)))
    while len(par) < K:
        par.append(int(rng.choice([-1] + list(range(len(par))))))
    return np.array(par, np.int32), main


@pytest.mark.parametrize("name,plen,K,kind", [
    ("tiny_gqa_bf16", 100, 16, "chain"), ("tiny_gqa_bf16", 236, 16, "chain"),
    ("tiny_hybrid_bf16", 100, 20, "tree"), ("tiny_gqa", 100, 16, "chain"),
    ("dense8b_l2", 120, 16, "chain"), ("hybrid27b_l4", 120, 32, "tree"),
    ("tiny_gqa_bf16", 100, 64, "tree"), ("dense8b_l2", 120, 64, "tree")])
@pytest.mark.parametrize("stream", [True, False])
def test_row_count_invariance(name, plen, K, kind, stream):
    """A verify pass of one request with at most 128 rows computes each row's
    logits with the same bits as a one-row pass (an AR step) at that row's
    position: the root row against the AR step at the committed length, and
    each main-path node against the AR step after committing the path up to
    it (token forcing).  Chains of 17 rows and trees of 21, 33 (the
    full-width 27B shape with two query groups) and 65 rows (the 8B tree:
    the GEMMs' two-tile shape, three query groups), attention streamed (the
    planner's choice) or one key split per workgroup (the debug flag); the
    236-token prompt crosses a 256-key boundary of the attention plan between
    the verify and the last AR step."""
    cfg, W = _setup(name)
    V = cfg["vocab"]
    eng = engine_for(cfg, W, max_ctx=512, max_nodes=K + 1)
    if not stream:
        eng.debug_flags(4)
    eng.prefill(0, synth.prompt_tokens(V, plen, 77))
    rng = np.random.default_rng(5)
    drafts = rng.integers(0, V, K).astype(np.int32)
    if kind == "chain":
        parents, main = np.arange(-1, K - 1, dtype=np.int32), list(range(K))
    else:
        parents, main = _main_path_tree(K, 6, rng)
    _, _, lg = eng.verify([0], [drafts], [parents], logits=True)
    rows = lg.cpu().numpy().copy()
    empty = np.zeros(0, np.int32)
    for j in range(5):
        _, _, l1 = eng.verify([0], [empty], [empty], logits=True)
        one = l1.cpu().numpy()[0].copy()
        ref = rows[0] if j == 0 else rows[main[j - 1] + 1]
        _say(name, kind, "streamed" if stream else "split", "step", j,
             float(np.max(np.abs(one - ref))))
        assert np.array_equal(one.view(np.uint32), ref.view(np.uint32)), j
        eng.commit([0], [[]], [int(drafts[main[j]])])
    eng.close()


# ------------------------------------------------- W12 weight storage

def _run_steps(eng, cfg, prompt, steps, seed, big=0):
    """Prefill, then verify + commit steps alternating chains and trees
    (every third step a chain of `big` nodes when big > 0); returns every
    pass's paths, bonus tokens and logits."""
    V = cfg["vocab"]
    rng = np.random.default_rng(seed)
    tree_par = np.array([-1, 0, 0, 1, 2, 3, -1, 6, 7, 4, 9, 5])
    first, lg = eng.prefill(0, prompt, logits=True)
    out = [(first, lg.cpu().numpy().copy())]
    for k in range(steps):
        if big and k % 3 == 2:
            toks, par = rng.integers(0, V, big), np.arange(-1, big - 1)
        elif k % 2:
            toks, par = rng.integers(0, V, 12), tree_par
        else:
            toks, par = rng.integers(0, V, 8), np.arange(-1, 7)
        paths, bonus, lg = eng.verify([0], [toks], [par], logits=True)
        out.append((paths, bonus, lg.cpu().numpy().copy()))
        eng.commit([0], paths, bonus)
    return out


def _assert_same(a, b):
    assert a[0][0] == b[0][0] and np.array_equal(a[0][1], b[0][1])
    for (pa, ba, la), (pb, bb, lb) in zip(a[1:], b[1:]):
        assert pa == pb and ba == bb
        assert np.array_equal(la, lb)


@pytest.mark.parametrize("name", ["tiny_gqa_bf16", "tiny_hybrid_bf16", "dense8b_l2"])
def test_w12_weights_give_bitwise_identical_results(name):
    """W12 storage restores every bf16 weight exactly, so logits, paths and
    bonus tokens equal those of bf16 storage bit for bit."""
    cfg, W = _setup(name)
    prompt = synth.prompt_tokens(cfg["vocab"], 90, 55)
    runs = []
    for fmt in ("native", "w12"):
        eng = engine_for(cfg, W, max_ctx=512, max_nodes=17, weight_format=fmt)
        runs.append(_run_steps(eng, cfg, prompt, 6, 55))
        eng.close()
    _assert_same(*runs)


def test_w12_exceptions():
    """Weights the 12-bit code cannot hold: exact zeros, negative zeros,
    bf16 subnormals and values far below their row's largest (a row with one
    large weight), at most 7 in any tile.  Results must still equal bf16
    storage bit for bit."""
    cfg, W0 = _setup("tiny_gqa_bf16")
    W = dict(W0)
    names = [n for n, _, k in synth.tensor_specs(cfg) if k == "mat" and n != "embed"]
    rng = np.random.default_rng(56)
    for i, n in enumerate(names):
        w = W[n].copy()                      # bf16 bit patterns (uint16)
        r, c = w.shape
        # one tile with exactly 7 exceptions (tile row t0 // 16, K-step 1)
        t0 = ((i * 16) % r) // 16 * 16
        full = (t0 // 16) * (c // 32) + 1
        sel = rng.choice(512, 7, replace=False)
        w[t0 + sel // 32, 32 + sel % 32] = 0
        # scattered exact zeros, negative zeros and subnormals, one per tile
        tiles = rng.choice((r // 16) * (c // 32), size=max(12, r * c // 4000),
                           replace=False)
        tiles = tiles[tiles != full]
        rr = (tiles // (c // 32)) * 16 + rng.integers(0, 16, tiles.size)
        cc = (tiles % (c // 32)) * 32 + rng.integers(0, 32, tiles.size)
        vals = np.where(np.arange(tiles.size) % 3 == 0, 0x0000,
                        np.where(np.arange(tiles.size) % 3 == 1, 0x8000,
                                 rng.integers(1, 0x7F, tiles.size)))
        w[rr, cc] = vals.astype(np.uint16)
        # one row (outside that tile) with a large weight: its small weights
        # leave the row's exponent window
        w[(t0 + 16 + 3 * i % 16) % r, 5] = 0x3F80   # 1.0
        W[n] = w
    prompt = synth.prompt_tokens(cfg["vocab"], 60, 56)
    runs = []
    for fmt in ("native", "w12"):
        # 47 drafts + root = 48 rows: the GEMMs at 3 row tiles (the other
        # loop shape)
        eng = engine_for(cfg, W, max_ctx=512, max_nodes=48, weight_format=fmt)
        runs.append(_run_steps(eng, cfg, prompt, 6, 56, big=47))
        eng.close()
    assert np.all(np.isfinite(runs[0][0][1]))
    _assert_same(*runs)


def _crowd(w, tile_row, kstep, n, rng, val=0):
    """Set n weights of one 16 x 32 tile of w (bf16 bits) to `val` (0: an
    exact zero, which W12 cannot hold in the window)."""
    sel = rng.choice(512, n, replace=False)
    w[tile_row * 16 + sel // 32, kstep * 32 + sel % 32] = val


def test_w12_crowded_tiles_spill_to_overflow_blocks():
    """Tiles with more exceptions than the 7-entry slot (8, 20 and 63, the
    most a tile holds) keep the rest in their overflow blocks; every GEMM
    shape that patches them (up to 32 rows: the compiler's loop; 36 and 48
    rows: the assembly block) must give results bitwise equal to bf16
    storage.  The crowded tiles sit in fused matrices (Wk inside QKV, the
    up half of gate/up) and in plain ones (O, down, LM head)."""
    cfg, W0 = _setup("tiny_gqa_bf16")
    W = dict(W0)
    rng = np.random.default_rng(57)
    for name, plants in (("layers.0.wk", [(1, 2, 8), (3, 5, 63)]),
                         ("layers.1.wu", [(0, 0, 20), (7, 3, 9)]),
                         ("layers.0.wo", [(2, 1, 63)]),
                         ("layers.1.wd", [(4, 9, 33)]),
                         ("lm_head", [(5, 4, 40), (100, 15, 8)])):
        w = W[name].copy()
        for tr, kb, n in plants:
            _crowd(w, tr, kb, n, rng)
        W[name] = w
    prompt = synth.prompt_tokens(cfg["vocab"], 60, 57)
    for big in (35, 47):
        runs = []
        for fmt in ("native", "w12"):
            eng = engine_for(cfg, W, max_ctx=512, max_nodes=48, weight_format=fmt)
            runs.append(_run_steps(eng, cfg, prompt, 6, 57, big=big))
            eng.close()
        _assert_same(*runs)


def test_w12_tile_over_capacity_is_rejected_and_retried():
    """A tile with more exceptions than the slot and its overflow block hold
    (64) does not fit W12: that load fails with SPEC_E_UNSUPPORTED, the
    error does not stick to the matrix (a retry with fitting weights and
    the fused partners load), and the results then equal bf16 storage."""
    from tree_verification_spec_amd import SpecError, SPEC_E_UNSUPPORTED, Engine
    import tree_verification_spec_amd._lib as L
    import torch
    cfg, W = _setup("tiny_gqa_bf16")
    specs = synth.tensor_specs(cfg)
    names = [n for n, _, _ in specs]
    bad_id = names.index("layers.0.wq")
    bad = W["layers.0.wq"].copy()
    _crowd(bad, 2, 3, 64, np.random.default_rng(3))
    eng = Engine(cfg, max_ctx=512, max_nodes=17, weight_format="w12")
    dev = eng.device

    def load(tid, a):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16
                             else np.ascontiguousarray(a)).to(dev)
        torch.cuda.synchronize(dev)
        L.spec_load_weights(eng.ctx, tid, t.data_ptr(), a.nbytes, 1)

    for tid, n in enumerate(names):
        if tid == bad_id:
            with pytest.raises(SpecError) as ei:
                load(tid, bad)
            assert ei.value.code == SPEC_E_UNSUPPORTED
        load(tid, W[n])
    prompt = synth.prompt_tokens(cfg["vocab"], 60, 58)
    got = _run_steps(eng, cfg, prompt, 4, 58)
    eng.close()
    ref_eng = engine_for(cfg, W, max_ctx=512, max_nodes=17, weight_format="native")
    ref = _run_steps(ref_eng, cfg, prompt, 4, 58)
    ref_eng.close()
    _assert_same(got, ref)


# ------------------------------------------------ two-level verification

def _view8(w):
    """The 8-bit view of bf16 weight bits, from the format's definition: per
    output row the base eb = max(0, largest exponent (255 counted as 254) -
    15); a weight whose exponent lies in [eb, eb + 15] keeps its sign,
    exponent and top 3 mantissa bits; any other keeps only its sign, with
    exponent eb and mantissa 0."""
    w = w.astype(np.int64)
    exp = (w >> 7) & 0xFF
    eb = np.maximum(np.minimum(exp.max(axis=1), 254) - 15, 0)[:, None]
    inwin = (exp >= eb) & (exp <= eb + 15) & (exp != 255)
    return np.where(inwin, w & 0xFFF0, (w & 0x8000) | (eb << 7)).astype(np.uint16)


def _lowp_setup():
    cfg, W = _setup("tiny_gqa_bf16")
    W8 = {n: (_view8(W[n]) if k == "mat" and n != "embed" else W[n])
          for n, _, k in synth.tensor_specs(cfg)}
    return cfg, W, W8


def test_lowp_pass_matches_oracle_on_8bit_view():
    """spec_verify_lowp = the model with every GEMM weight replaced by its
    8-bit view, over the exact committed cache; it accepts nothing."""
    from oracle.verify import verify_single_pass
    from tree_verification_spec_amd import SpecError, SPEC_E_STATE
    cfg, W, W8 = _lowp_setup()
    V = cfg["vocab"]
    orc, orc8 = oracle_for(cfg, W), oracle_for(cfg, W8)
    eng = engine_for(cfg, W, max_ctx=512, max_nodes=13, weight_format="w12_lowp")
    prompt = synth.prompt_tokens(V, 50, 71)
    S, L, M, st = ar_greedy(orc, prompt, 1)
    first = eng.prefill(0, prompt)
    assert first == S[0] or M[0] < NEAR_TIE
    eng.force_root(0, int(S[0]))
    rng = np.random.default_rng(71)
    for kind, K in (("chain", 8), ("tree", 12)):
        toks = rng.integers(0, V, K)
        par = (np.arange(-1, K - 1) if kind == "chain" else
               np.array([-1, 0, 0, 1, 2, 3, -1, 6, 7, 4, 9, 5])[:K])
        state0 = eng.state(0)
        paths, bonus, lg = eng.verify([0], [toks], [par], logits=True, lowp=True)
        lg = lg.cpu().numpy()
        ref, A, rpath, rbonus = verify_single_pass(orc8, st, int(S[0]), toks, par)
        for i in range(K + 1):
            assert np.max(np.abs(lg[i] - ref[i])) <= logit_tol(cfg["dtype"], ref[i]), (kind, i)
        if all(top2_margin(ref[i]) >= NEAR_TIE for i in range(K + 1)):
            assert paths[0] == rpath and bonus[0] == rbonus
        assert eng.state(0) == state0
        with pytest.raises(SpecError) as e:
            eng.commit([0], paths, bonus)
        assert e.value.code == SPEC_E_STATE
    # the 8-bit view is not the exact model: some logits must differ
    ref_exact, *_ = verify_single_pass(orc, st, int(S[0]), toks, par)
    assert np.max(np.abs(ref_exact - ref)) > 10 * logit_tol(cfg["dtype"], ref_exact[0])
    eng.close()


def test_two_level_steps_emit_ar_tokens():
    """Two-level steps: the low-precision pass turns 4 drafts into a
    candidate chain (its accepted drafts and its bonus token), the drafter
    continues 3 positions from the chain's end, and one exact pass verifies
    the whole chain.  Emitted tokens equal the oracle's greedy run."""
    cfg, W, _ = _lowp_setup()
    V = cfg["vocab"]
    orc = oracle_for(cfg, W)
    n_gen, K1, K2, alpha = 48, 4, 3, 0.7
    eng = engine_for(cfg, W, max_ctx=512, max_nodes=K1 + K2 + 2, weight_format="w12_lowp")
    prompt = synth.prompt_tokens(V, 40, 72)
    S, L, M, _ = ar_greedy(orc, prompt, n_gen)
    first = eng.prefill(0, prompt)
    if first != S[0]:
        assert M[0] < NEAR_TIE
        eng.force_root(0, int(S[0]))
    g, step, ties, cand_total = 1, 0, 0, 0
    while g < n_gen:
        d1, p1 = synth.chain_drafts(S, g, K1, alpha, V, 72, 0, step)
        lpath, lbonus = eng.verify([0], [d1], [p1], lowp=True)
        cand = [int(d1[p]) for p in lpath[0]] + [lbonus[0]]
        d2, _ = synth.chain_drafts(S, g + len(cand), K2, alpha, V, 73, 0, step)
        chain = np.array(cand + [int(t) for t in d2], np.int64)
        paths, bonus = eng.verify([0], [chain], [np.arange(-1, len(chain) - 1)])
        emitted = [int(chain[p]) for p in paths[0]] + [bonus[0]]
        n_ok = 0
        for j, t in enumerate(emitted):
            if g + j >= n_gen or t != S[g + j]:
                break
            n_ok += 1
        if n_ok < len(emitted) and g + n_ok < n_gen:
            assert M[g + n_ok] < NEAR_TIE, (step, g, emitted, S[g:g + 8])
            ties += 1
            keep = paths[0][:n_ok]
            eng.commit([0], [keep], [int(S[g + n_ok])])
            g += len(keep) + 1
        else:
            eng.commit([0], paths, bonus)
            g += len(emitted)
        cand_total += len(cand)
        step += 1
    _say("two-level steps", step, "tokens", g, "candidate tokens", cand_total, "ties", ties)
    assert ties <= 3
    assert g / step > 1.5
    eng.close()


# ------------------------------------- matches off the main branch, ties

def _branch_trees(S, g, V, rng):
    """Trees whose matching tokens sit on more than one branch (drafts,
    draft parents with -1 = the root, and the accepted draft path the rule
    gives when the target's greedy tokens are S[g], S[g+1], S[g+2]).
    deep: two sibling copies of S[g]; the second one's branch reaches depth
    3, the first one's stops at depth 2, so the walk must take the second
    (non-main) branch.  equal: both branches reach depth 2; the lower node
    index (on the second sibling's branch) wins."""
    wrong = lambda t: int((t + 1 + rng.integers(0, V - 1)) % V)
    a, b, c = int(S[g]), int(S[g + 1]), int(S[g + 2])
    return {"deep": ([a, a, wrong(a), b, b, wrong(c), c], [-1, -1, -1, 1, 0, 4, 3], [1, 3, 6]),
            "equal": ([a, a, b, b, wrong(c)], [-1, -1, 1, 0, 3], [1, 2])}


@pytest.mark.parametrize("name", ["tiny_gqa_bf16", "tiny_hybrid_bf16", "dense8b_l2"])
def test_off_main_branch_accepted_and_compacted(name):
    """The accepted path runs through a second sibling (deeper branch, then
    equal depth with the lower index): the walk's choice, every row's logits
    against the oracle's tree pass, and then chain steps whose logits
    depend on the compacted KV cache and the committed recurrent state of
    that branch, against the oracle's AR logits."""
    from oracle import accept_path
    cfg, W = _setup(name)
    V = cfg["vocab"]
    orc = oracle_for(cfg, W)
    prompt = synth.prompt_tokens(V, 80, 61)
    n = 40
    S, L, M, _ = ar_greedy(orc, prompt, n)
    eng = engine_for(cfg, W, max_ctx=512, max_nodes=17)
    first = eng.prefill(0, prompt)
    assert first == S[0]
    ost = orc.new_state()
    orc.prefill(ost, prompt)
    rng = np.random.default_rng(62)
    g, worst, branch_steps = 1, 0.0, 0
    for kind in ("deep", "equal", "deep"):
        toks, par, want = _branch_trees(S, g, V, rng)[kind]
        nodes = [int(S[g - 1])] + toks
        npar = [-1] + [p + 1 for p in par]
        ref = orc.forward(ost, nodes, npar)
        opath, obonus = accept_path(nodes, npar, ref.argmax(axis=1))
        paths, bonus, lg = eng.verify([0], [toks], [par], logits=True)
        lg = lg.cpu().numpy()
        for i in range(len(nodes)):
            worst = max(worst, float(np.max(np.abs(lg[i] - ref[i]))) / logit_tol(cfg["dtype"], ref[i]))
        got = [p + 1 for p in paths[0]]
        assert got == opath, (kind, got, opath)
        branch_steps += [p - 1 for p in opath] == want
        pos = g + len(opath)            # the bonus position
        root = int(bonus[0])
        if root != obonus or obonus != int(S[pos]):
            assert M[pos] < NEAR_TIE, (kind, root, obonus, int(S[pos]))
            root = int(S[pos])
        eng.commit([0], paths, [root])
        for t in [int(S[g - 1])] + [toks[p] for p in paths[0]]:
            orc.decode(ost, t)
        g = pos + 1
    assert branch_steps == 3, "the designed branches were not the accepted ones"
    # chain steps after the branch commits
    step = 0
    while g < n - 10:
        toks, par = synth.chain_drafts(S, g, 8, 0.7, V, 61, 0, step)
        paths, bonus, lg = eng.verify([0], [toks], [par], logits=True)
        lg = lg.cpu().numpy()
        em = [int(toks[p]) for p in paths[0]] + [int(bonus[0])]
        rows = [0] + [p + 1 for p in paths[0]]
        n_ok = 0
        while n_ok < len(em) and em[n_ok] == S[g + n_ok]:
            n_ok += 1
        for i in range(min(len(rows), n_ok + 1)):
            worst = max(worst, float(np.max(np.abs(lg[rows[i]] - L[g + i]))) /
                        logit_tol(cfg["dtype"], L[g + i]))
        if n_ok < len(em):
            assert M[g + n_ok] < NEAR_TIE, (g + n_ok, em[n_ok], S[g + n_ok])
            keep = paths[0][:n_ok] if n_ok < len(paths[0]) else paths[0]
            eng.commit([0], [keep], [int(S[g + len(keep)])])
            g += len(keep) + 1
        else:
            eng.commit([0], paths, bonus)
            g += len(em)
        step += 1
    _say(f"{name}: max logit error {worst:.3f} x tolerance")
    assert worst <= 1.0
    eng.close()


def test_planted_argmax_ties_take_the_lowest_index():
    """Exact ties planted in the LM head (a lower-index copy of a token's
    row, once in the same column tile and once in another column block):
    wherever the copied token would win, the lower index must be emitted,
    bit-exactly, with no near-tie exemption."""
    cfg, W0 = _setup("tiny_gqa")
    V = cfg["vocab"]
    prompt = synth.prompt_tokens(V, 64, 65)
    S0, _, _, _ = ar_greedy(oracle_for(cfg, W0), prompt, 24)
    t1 = next(int(t) for t in S0 if t % 16 != 0)
    lm = W0["lm_head"].copy()
    lm[t1 - 1] = lm[t1]          # same 16-column tile
    S1, _, _, _ = ar_greedy(oracle_for(cfg, dict(W0, lm_head=lm)), prompt, 24)
    t2 = next(int(t) for t in S1 if t >= 256 and abs(int(t) - t1) > 2
              and t % 128 not in (t1, t1 - 1))
    lm[t2 % 128] = lm[t2]        # the first column block
    W = dict(W0, lm_head=lm)
    orc = oracle_for(cfg, W)
    S, L, M, _ = ar_greedy(orc, prompt, 48)
    n_ties = int(np.sum(M == 0.0))
    assert n_ties >= 2 and (t1 - 1 in S) and (t2 % 128 in S), (n_ties, t1, t2)
    eng = engine_for(cfg, W, max_ctx=512, max_nodes=5)
    w = dict(K=4, alpha=0.7)
    rep = protocol_f(eng, cfg, orc, prompt, 48, w, "chain", cfg_index=65,
                     oracle_ref=(S, L, M))
    _say(rep, "exact ties in the reference:", n_ties)
    assert rep.first_bad is None and rep.near_tie_mismatch == 0, rep
    assert rep.max_logit_err <= 1.0
    eng.close()


@pytest.mark.parametrize("name", ["tiny_hybrid", "tiny_hybrid_bf16"])
def test_recurrent_walk_deep_trees_and_mixed_passes(name):
    """The recurrent layers walk trees depth-first with the root path's
    states in registers when every node of the pass is at most 14 deep, and
    recompute each node's state along its root path otherwise.  Cases: a
    tree 30 deep (a spine with side branches), a pass mixing that tree with
    a 24-long chain, a pass mixing a shallow tree with a 20-long chain (deep
    class because of the chain), a shallow tree alone, and the two sides of
    the class boundary (chains of 14 and 15 drafts beside a shallow tree);
    every row's logits against the oracle's tree pass from the same
    committed state."""
    cfg, W = _setup(name)
    V = cfg["vocab"]
    orc = oracle_for(cfg, W)
    eng = engine_for(cfg, W, max_requests=2, max_ctx=512, max_nodes=40, max_rows=80)
    rng = np.random.default_rng(71)
    ost, roots = [], []
    for r in range(2):
        prompt = synth.prompt_tokens(V, 40, 70 + r)
        roots.append(eng.prefill(r, prompt))
        st = orc.new_state()
        orc.prefill(st, prompt)
        ost.append(st)
    # drafts: parents (-1 = the root)
    spine = list(range(-1, 29))                       # 30 drafts, depth 30
    deep = spine + [2, 2, 9, 31, 19, 20, 33]          # side branches at depths 4, 11, 21
    shallow = [-1, -1, 0, 0, 1, 2, 3, 3, 4, -1, 9]    # depth <= 4
    chain = lambda k: list(range(-1, k - 1))
    cases = [[(0, deep)], [(0, deep), (1, chain(24))], [(0, shallow), (1, chain(20))],
             [(0, shallow)], [(0, shallow), (1, chain(14))], [(0, shallow), (1, chain(15))]]
    worst = 0.0
    for case in cases:
        reqs = [r for r, _ in case]
        par = [np.array(p, np.int32) for _, p in case]
        toks = [rng.integers(0, V, len(p)).astype(np.int32) for p in par]
        paths, bonus, lg = eng.verify(reqs, toks, par, logits=True)
        lg = lg.cpu().numpy()
        row = 0
        for k, r in enumerate(reqs):
            nodes = np.concatenate([[roots[r]], toks[k]])
            npar = np.concatenate([[-1], par[k] + 1])
            ref = orc.forward(ost[r], nodes, npar)
            for i in range(len(nodes)):
                err = float(np.max(np.abs(lg[row + i] - ref[i])))
                worst = max(worst, err / logit_tol(cfg["dtype"], ref[i]))
            row += len(nodes)
    _say(f"{name}: max logit error {worst:.3f} x tolerance")
    assert worst <= 1.0
    eng.close()
