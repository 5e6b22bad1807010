"""Pins of the oracle's whole model and of its tree verification.

* the dense model against an independent library implementation of the same
  architecture (transformers' Llama: RMSNorm, rotate-half RoPE, GQA, SwiGLU,
  untied LM head, no biases);
* incremental (KV cache) decoding against full recomputation of each prefix;
* the single tree-masked pass against per-node brute force;
* the lossless invariant: tree verification accepts exactly the AR prefix.
"""

import os

import numpy as np
import pytest
import torch

import synth
from oracle import (Model, ar_greedy, verify_single_pass, verify_bruteforce,
                    accept_path, top2_margin)


def _model(name, weights_cache=None):
    cfg = synth.model_config(name)
    w = weights_cache(name) if weights_cache else synth.make_weights(cfg)
    return Model(cfg, w, max_pos=4096)


# ------------------------------------------------ library pin (transformers)

@pytest.mark.parametrize("name", ["tiny", "tiny_gqa"])
def test_dense_model_matches_transformers_llama(name):
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = synth.model_config(name)
    w = synth.make_weights(cfg)
    hcfg = LlamaConfig(
        vocab_size=cfg["vocab"], hidden_size=cfg["d_model"],
        intermediate_size=cfg["ffn_dim"], num_hidden_layers=cfg["n_layers"],
        num_attention_heads=cfg["n_heads"],
        num_key_value_heads=cfg["n_kv_heads"], head_dim=cfg["head_dim"],
        rms_norm_eps=cfg["rms_eps"], rope_theta=cfg["rope_theta"],
        max_position_embeddings=4096, tie_word_embeddings=False,
        attention_bias=False, mlp_bias=False, hidden_act="silu")
    hcfg._attn_implementation = "eager"
    hf = LlamaForCausalLM(hcfg).eval()
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32))
    sd = {"model.embed_tokens.weight": T(w["embed"]),
          "model.norm.weight": T(w["final_norm"]),
          "lm_head.weight": T(w["lm_head"])}
    names = {"attn_norm": "input_layernorm", "wq": "self_attn.q_proj",
             "wk": "self_attn.k_proj", "wv": "self_attn.v_proj",
             "wo": "self_attn.o_proj", "ffn_norm": "post_attention_layernorm",
             "wg": "mlp.gate_proj", "wu": "mlp.up_proj", "wd": "mlp.down_proj"}
    for i in range(cfg["n_layers"]):
        for ours, theirs in names.items():
            sd[f"model.layers.{i}.{theirs}.weight"] = T(w[f"layers.{i}.{ours}"])
    missing, unexpected = hf.load_state_dict(sd, strict=False)
    assert not unexpected and all("rotary" in m for m in missing), (missing,
                                                                    unexpected)
    toks = synth.prompt_tokens(cfg["vocab"], 48, 90)
    with torch.no_grad():
        ref = hf(torch.from_numpy(toks.astype(np.int64))[None]).logits[0].numpy()
    m = Model(cfg, w, max_pos=4096)
    st = m.new_state()
    got = m.append(st, toks)
    assert np.max(np.abs(got - ref)) < 5e-5, np.max(np.abs(got - ref))


# ----------------------------------------- incremental vs recompute (P1)

@pytest.mark.parametrize("name", ["tiny", "tiny_gqa", "tiny_hybrid",
                                  "tiny_gqa_bf16", "tiny_hybrid_bf16"])
def test_incremental_equals_full_recompute(name):
    m = _model(name)
    V = m.cfg["vocab"]
    prompt = synth.prompt_tokens(V, 23, 91)
    S, L, _, _ = ar_greedy(m, prompt, 6)
    # bf16 models: a one-ulp flip of a bf16-rounded activation (different
    # BLAS blocking for different row counts) moves logits by ~1e-2 std;
        # the fp32 variants pin the same code paths at 1e-5
    for t in range(6):
        tol = 1e-5 if m.cfg["dtype"] == "fp32" else 2e-2 * np.std(L[t])
        st = m.new_state()
        full = m.append(st, np.concatenate([prompt, S[:t]]))[-1]
        assert np.max(np.abs(full - L[t])) < tol, (t, np.max(np.abs(full - L[t])))


def test_chunked_prefill_equals_one_pass():
    m = _model("tiny_hybrid")
    prompt = synth.prompt_tokens(m.cfg["vocab"], 40, 92)
    a = m.prefill(m.new_state(), prompt, chunk=1000)
    b = m.prefill(m.new_state(), prompt, chunk=7)
    assert np.max(np.abs(a - b)) < 1e-5


# ---------------------------------------------- single pass vs brute (P3)

def _random_tree(rng, K):
    parents = np.array([-1] + [int(rng.integers(-1, i)) for i in range(1, K)],
                       np.int32)
    return parents


@pytest.mark.parametrize("name", ["tiny", "tiny_gqa", "tiny_hybrid",
                                  "tiny_gqa_bf16", "tiny_hybrid_bf16"])
def test_tree_single_pass_equals_bruteforce(name):
    m = _model(name)
    V = m.cfg["vocab"]
    rng = np.random.default_rng(11)
    st = m.new_state()
    m.prefill(st, synth.prompt_tokens(V, 19, 93))
    drafts = rng.integers(0, V, 9).astype(np.int32)
    parents = _random_tree(rng, 9)
    l1, A1, p1, b1 = verify_single_pass(m, st, 5, drafts, parents)
    l2, A2, p2, b2 = verify_bruteforce(m, st, 5, drafts, parents)
    tol = 1e-5 if m.cfg["dtype"] == "fp32" else 2e-2 * np.std(l2)
    assert np.max(np.abs(l1 - l2)) < tol
    assert st.n == 19   # verification leaves the committed state alone


# ------------------------------------------------- lossless invariant (P2)

def _planted_tree(rng, S, g, K, plant_len, V):
    """Random topology with the AR continuation planted along one path of
    length plant_len; every other node avoids the AR token at its depth."""
    parents = _random_tree(rng, K)
    depth = np.zeros(K, int)
    for i in range(K):
        depth[i] = 1 if parents[i] < 0 else depth[parents[i]] + 1
    # pick a deepest-enough node and plant along its path
    cand = [i for i in range(K) if depth[i] >= plant_len]
    toks = np.zeros(K, np.int32)
    on_path = set()
    if plant_len > 0 and cand:
        v = int(rng.choice(cand))
        chain = []
        while v != -1:
            chain.append(v)
            v = parents[v]
        chain.reverse()
        on_path = set(chain[:plant_len])
    for i in range(K):
        tgt = int(S[g - 1 + depth[i]]) if g - 1 + depth[i] < len(S) else None
        if i in on_path:
            toks[i] = tgt
        else:
            t = int(rng.integers(0, V - 1))
            toks[i] = t + (tgt is not None and t >= tgt)
    return toks, parents, (len(on_path) if on_path else 0)


@pytest.mark.parametrize("name", ["tiny", "tiny_hybrid_bf16"])
def test_tree_verification_accepts_exactly_the_ar_prefix(name):
    m = _model(name)
    V = m.cfg["vocab"]
    prompt = synth.prompt_tokens(V, 17, 94)
    S, L, M, _ = ar_greedy(m, prompt, 14)
    rng = np.random.default_rng(12)
    st = m.new_state()
    m.prefill(st, prompt)
    # after prefill the pending root is S[0], g = 1 token emitted
    for plant in (0, 1, 2, 3, 4):
        toks, parents, planted = _planted_tree(rng, S, 1, 10, plant, V)
        _, _, path, bonus = verify_single_pass(m, st, int(S[0]), toks, parents)
        emitted = [int(toks[p]) for p in path] + [bonus]
        assert len(path) == planted
        assert emitted == [int(s) for s in S[1:len(emitted) + 1]]


def test_chain_special_cases():
    m = _model("tiny")
    V = m.cfg["vocab"]
    prompt = synth.prompt_tokens(V, 12, 95)
    S, L, _, _ = ar_greedy(m, prompt, 10)
    st = m.new_state()
    m.prefill(st, prompt)
    chain = lambda k: np.arange(-1, k - 1, dtype=np.int32)
    # alpha = 1: every draft accepted, bonus = the next AR token
    _, _, path, bonus = verify_single_pass(m, st, int(S[0]), S[1:6], chain(5))
    assert path == [0, 1, 2, 3, 4] and bonus == S[6]
    # alpha = 0: nothing accepted
    wrong = (S[1:6] + 1) % V
    _, _, path, bonus = verify_single_pass(m, st, int(S[0]), wrong, chain(5))
    assert path == [] and bonus == S[1]
    # K = 0 equals one AR step (same logits as the AR run)
    lg, A, path, bonus = verify_single_pass(m, st, int(S[0]), [], [])
    assert path == [] and bonus == S[1]
    assert np.max(np.abs(lg[0] - L[1])) < 1e-5
    # a chain written as a general tree gives the same answer
    _, _, p2, b2 = verify_single_pass(m, st, int(S[0]),
                                      np.array([S[1], S[2], 7], np.int32),
                                      np.array([-1, 0, 1], np.int32))
    assert p2 == [0, 1] and b2 == (S[3] if S[3] != 7 else b2)
    # a star accepts at most one draft
    star = np.array([(S[1] + 3) % V, S[1], S[2]], np.int32)
    _, _, p3, b3 = verify_single_pass(m, st, int(S[0]), star,
                                      np.array([-1, -1, -1], np.int32))
    assert p3 == [1] and b3 == S[2]


def test_duplicate_subtrees_and_renumbering():
    """Equal tokens on two sibling branches: the lower index wins, emitted
    tokens are unchanged; any topological renumbering gives the same text."""
    m = _model("tiny_gqa")
    V = m.cfg["vocab"]
    prompt = synth.prompt_tokens(V, 15, 96)
    S, _, _, _ = ar_greedy(m, prompt, 8)
    st = m.new_state()
    m.prefill(st, prompt)
    toks = np.array([S[1], S[1], S[2], S[2], S[3]], np.int32)
    par = np.array([-1, -1, 0, 1, 3], np.int32)
    _, _, path, bonus = verify_single_pass(m, st, int(S[0]), toks, par)
    # branch 1 -> 3 -> 4 is deeper (3 matched) than 0 -> 2 (2 matched)
    assert path == [1, 3, 4] and bonus == S[4]
    # renumber: reverse the two branches
    toks2 = np.array([S[1], S[2], S[3], S[1], S[2]], np.int32)
    par2 = np.array([-1, 0, 1, -1, 3], np.int32)
    _, _, path2, bonus2 = verify_single_pass(m, st, int(S[0]), toks2, par2)
    assert [int(toks2[p]) for p in path2] + [bonus2] == \
        [int(toks[p]) for p in path] + [bonus]
    # equal depth tie: lower node index wins
    toks3 = np.array([S[1], S[1]], np.int32)
    _, _, p3, _ = verify_single_pass(m, st, int(S[0]), toks3,
                                     np.array([-1, -1], np.int32))
    assert p3 == [0]


def test_accept_path_hand_cases():
    # nodes: 0 root; 1,2 children of 0; 3 child of 1; 4 child of 2; 5 child of 4
    toks = [9, 5, 5, 6, 6, 8]
    par = [-1, 0, 0, 1, 2, 4]
    A = [5, 6, 6, 1, 8, 3]
    path, bonus = accept_path(toks, par, A)
    assert path == [2, 4, 5] and bonus == 3
    A = [5, 6, 7, 1, 8, 3]            # node 4 no longer matches A(2)
    path, bonus = accept_path(toks, par, A)
    assert path == [1, 3] and bonus == 1
    A = [4, 6, 7, 1, 8, 3]            # nothing matches the root's choice
    path, bonus = accept_path(toks, par, A)
    assert path == [] and bonus == 4


def _golden_accept_cases():
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                        "accept_path_cases.txt")
    cases, cur = [], None
    for line in open(path):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {"name": vals[0]}
            cases.append(cur)
        elif key in ("path",):
            cur[key] = [] if vals == ["-"] else [int(v) for v in vals]
        elif key == "bonus":
            cur[key] = int(vals[0])
        else:
            cur[key] = [int(v) for v in vals]
    return cases


def _accept_by_enumeration(toks, par, A):
    """Every root-to-node path, kept when each node's token equals its
    parent's argmax; the longest wins, then the one ending at the lowest
    node index."""
    best = (0, 0)
    for end in range(len(toks)):
        chain, v = [], end
        while v != 0:
            chain.append(v)
            v = par[v]
        if all(toks[c] == A[par[c]] for c in chain) and \
                (len(chain), -end) > (best[0], -best[1]):
            best = (len(chain), end)
    chain, v = [], best[1]
    while v != 0:
        chain.append(v)
        v = par[v]
    return chain[::-1], A[best[1]]


def test_accept_path_golden_cases():
    cases = _golden_accept_cases()
    assert len(cases) >= 10
    for c in cases:
        got = accept_path(c["tokens"], c["parents"], c["argmax"])
        assert got == (c["path"], c["bonus"]), c["name"]
        assert _accept_by_enumeration(c["tokens"], c["parents"], c["argmax"]) == \
            (c["path"], c["bonus"]), c["name"]


def test_top2_margin():
    assert abs(top2_margin(np.array([0.1, 3.0, 2.5, -1.0], np.float32)) - 0.5) < 1e-6
    assert top2_margin(np.array([2.0, 2.0, 1.0], np.float32)) == 0.0


# ----------------------------------------------------- full-width variants

@pytest.mark.slow
@pytest.mark.parametrize("name", ["dense8b_l2", "hybrid27b_l4"])
def test_full_width_variants(name, weights_cache):
    """Real d, heads, FFN and vocabulary with few layers: incremental ==
    recompute, single pass == brute force, and the logit spread is near
    sqrt(d) * 0.02 (a sanity range, not a pass/fail value of the pages)."""
    m = _model(name, weights_cache)
    V = m.cfg["vocab"]
    prompt = synth.prompt_tokens(V, 9, 97)
    S, L, M, st = ar_greedy(m, prompt, 4)
    st = m.new_state()
    full = m.append(st, np.concatenate([prompt, S[:2]]))[-1]
    assert np.max(np.abs(full - L[2])) < 2e-2 * np.std(L[2])
    std = float(np.std(L[0]))
    expect = (m.cfg["d_model"] ** 0.5) * 0.02
    assert 0.5 * expect < std < 2.0 * expect
    st = m.new_state()
    m.prefill(st, prompt)
    drafts = np.array([S[1], S[2], 3, 4], np.int32)
    parents = np.array([-1, 0, -1, 2], np.int32)
    l1, _, p1, b1 = verify_single_pass(m, st, int(S[0]), drafts, parents)
    l2, _, p2, b2 = verify_bruteforce(m, st, int(S[0]), drafts, parents)
    assert np.max(np.abs(l1 - l2)) < 2e-2 * std
    assert p1 == p2 == [0, 1] and b1 == b2 == S[3]
