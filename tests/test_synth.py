"""Input generators: determinism, topology rules and the closed-form
acceptance law of the synthesised drafts (checked with the oracle's
acceptance walk on a stand-in target whose greedy choice is the reference
sequence)."""

import math

import numpy as np
import pytest

import synth
from oracle import accept_path


def test_weights_deterministic_and_distribution():
    cfg = synth.model_config("tiny")
    a = synth.make_weights(cfg, threads=4)
    b = synth.make_weights(cfg, threads=1)
    for k in a:
        assert np.array_equal(a[k], b[k])
    e = a["embed"].astype(np.float64)
    assert abs(e.mean()) < 1e-3 and abs(e.std() - 0.02) < 2e-4
    assert np.all(a["final_norm"] == 1.0)


def test_bf16_weights_are_rounded_values():
    import torch
    cfg = synth.model_config("tiny_gqa_bf16")
    w = synth.make_weights(cfg)
    assert w["embed"].dtype == np.uint16
    f = synth.bf16_bits_to_f32(w["layers.0.wq"])
    assert abs(f.std() - 0.02) < 5e-4
    assert np.all(w["layers.1.ffn_norm"] == 0x3F80)
    # first chunk of the first matrix reproduces from its definition
    rng = np.random.default_rng([cfg["seed_w"], 0, 0])
    x = rng.standard_normal(cfg["vocab"] * cfg["d_model"], dtype=np.float32)
    x *= np.float32(0.02)
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(bits.view(np.uint16).reshape(w["embed"].shape),
                          w["embed"])


def test_tensor_specs_shapes():
    c = synth.model_config("hybrid27b")
    specs = synth.tensor_specs(c)
    names = [s[0] for s in specs]
    assert names[0] == "embed" and names[-1] == "lm_head"
    shapes = dict((s[0], s[1]) for s in specs)
    assert shapes["layers.0.w_in"] == (15488, 5120)
    assert shapes["layers.3.wq"] == (40 * 128, 5120)
    n = sum(int(np.prod(s[1])) for s in specs if s[2] == "mat")
    assert abs(n / 1e9 - 24.74) < 0.01
    c8 = synth.model_config("dense8b")
    n8 = sum(int(np.prod(s[1])) for s in synth.tensor_specs(c8) if s[2] == "mat")
    assert abs(n8 / 1e9 - 8.19) < 0.01


def test_tree_topology_rules():
    B = (4, 3, 2, 2, 1, 1, 1, 1)
    for step in range(20):
        parent, depth, main = synth.tree_topology(64, B, 8, 2, step)
        assert len(parent) == 64
        assert np.all(parent < np.arange(64))
        assert depth.max() == 8 and np.all(depth >= 1)
        assert main.sum() == 8
        kids = {}
        for i, p in enumerate(parent):
            kids[p] = kids.get(p, 0) + 1
        for p, n in kids.items():
            dp = 0 if p < 0 else depth[p]
            assert n <= B[dp]
        a, b, c = synth.tree_topology(64, B, 8, 2, step)
        assert np.array_equal(a, parent)


def _simulate(kind, alpha, K, steps, V=1000):
    """Acceptance with a stand-in target whose greedy token after a node at
    depth j is S[g-1+j+1]."""
    S = np.random.default_rng(0).integers(0, V, 100000).astype(np.int32)
    g, counts = 1, []
    B = (4, 3, 2, 2, 1, 1, 1, 1)
    for step in range(steps):
        if kind == "chain":
            toks, par = synth.chain_drafts(S, g, K, alpha, V, 9, 0, step)
        else:
            toks, par = synth.tree_drafts(S, g, K, B, 8, alpha, V, 9, 0, step)
        nt = np.concatenate([[S[g - 1]], toks])
        np_ = np.concatenate([[-1], par + 1])
        depth = np.zeros(len(nt), int)
        for i in range(1, len(nt)):
            depth[i] = depth[np_[i]] + 1
        A = [int(S[g - 1 + depth[i] + 1]) for i in range(len(nt))]
        path, bonus = accept_path(nt, np_, A)
        emitted = [int(nt[p]) for p in path] + [bonus]
        assert emitted == [int(s) for s in S[g:g + len(emitted)]]
        counts.append(len(emitted))
        g += len(emitted)
    return np.array(counts)


@pytest.mark.parametrize("kind,alpha,K,expect", [
    ("chain", 0.7, 4, 2.773), ("chain", 0.5, 16, 2.000),
    ("chain", 0.9, 16, 8.332), ("tree", 0.8, 64, 4.329),
    ("tree", 0.8, 32, 4.329)])
def test_acceptance_law_closed_form(kind, alpha, K, expect):
    depth = K if kind == "chain" else 8
    e = synth.expected_tokens_per_step(alpha, depth)
    assert abs(e - expect) < 1e-3
    # exact law P(m = j) = alpha^j (1 - alpha), P(m = depth) = alpha^depth
    p = np.array([alpha ** j * (1 - alpha) for j in range(depth)]
                 + [alpha ** depth])
    var = float(np.sum(p * (np.arange(depth + 1) + 1 - e) ** 2))
    n = 600
    c = _simulate(kind, alpha, K, n)
    assert abs(c.mean() - e) < 3 * math.sqrt(var / n), (c.mean(), e)


def test_batched_mix_and_prompts():
    ctx, alpha = synth.batched_mix(32, 512, 4096, 0.4, 0.9)
    assert ctx.min() >= 512 and ctx.max() <= 4096 and len(ctx) == 32
    assert alpha.min() >= 0.4 and alpha.max() <= 0.9
    p = synth.prompt_tokens(151936, 2048, 1)
    assert p.max() < 151936 and p.min() >= 0
    assert np.array_equal(p, synth.prompt_tokens(151936, 2048, 1))
