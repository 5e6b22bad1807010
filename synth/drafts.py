"""Prompts, draft chains, draft trees and the batched request mix.

There is no trained drafter: drafts are synthesised from a reference greedy
sequence ``S`` (the target's own autoregressive continuation) with a
controlled per-position match probability ``alpha``, so the acceptance length
can be swept.  Tree topologies follow the best-first construction the
SpecPilot pages describe: candidates are ranked by the log-probability of the
child given its parent and the nodes with the highest cumulative path score
are kept up to a node budget (besthub.dev article, "(2) Best-first Tree
Verification for Hybrid Architectures").

Index convention: ``S[0]`` is the first generated token (from prefill).  With
``g`` tokens emitted so far the pending root is ``S[g-1]``; a draft node at
depth ``j`` (the root has depth 0) should carry ``S[g-1+j]`` to be accepted.
"""

import heapq

import numpy as np


def prompt_tokens(vocab, length, cfg_index, req=0):
    rng = np.random.default_rng([100, cfg_index, req])
    return rng.integers(0, vocab, size=length, dtype=np.int64).astype(np.int32)


def _not_equal(rng, vocab, avoid):
    """Uniform over [0, vocab) minus {avoid} (any value when avoid is None)."""
    if avoid is None:
        return int(rng.integers(0, vocab))
    t = int(rng.integers(0, vocab - 1))
    return t + (t >= avoid)


def _target(S, g, depth):
    i = g - 1 + depth
    return int(S[i]) if 0 <= i < len(S) else None


def chain_drafts(S, g, K, alpha, vocab, cfg_index, req, step):
    """K draft tokens; parent_idx is the chain [-1, 0, 1, ..., K-2]."""
    rng = np.random.default_rng([200, cfg_index, req, step])
    hit = rng.random(K) < alpha
    toks = np.empty(K, np.int32)
    for j in range(1, K + 1):
        tgt = _target(S, g, j)
        if tgt is not None and hit[j - 1]:
            toks[j - 1] = tgt
        else:
            toks[j - 1] = _not_equal(rng, vocab, tgt)
    parents = np.arange(-1, K - 1, dtype=np.int32)
    return toks, parents


def tree_topology(budget, branching, max_depth, cfg_index, step):
    """Best-first draft tree.

    Returns (parent_idx[budget], depth[budget], main[budget]) for the draft
    nodes (the root is implicit, parent -1), in descending score order.
    ``main`` marks the forced rank-0 chain.
    """
    rng = np.random.default_rng([400, cfg_index, step])
    # node table: (score, parent_node, depth, rank, is_main); node 0 = root
    nodes = [(0.0, -1, 0, 0, True)]
    child_q = {}

    def expand(v):
        dep = nodes[v][2]
        if dep >= max_depth or dep >= len(branching):
            child_q[v] = np.zeros(0)
            return
        b = branching[dep]
        q = np.sort(rng.dirichlet(np.ones(b + 1)))[::-1]
        child_q[v] = q[:b]

    # forced main path (rank-0 chain) down to max_depth
    expand(0)
    v = 0
    while len(child_q[v]) > 0 and len(nodes) - 1 < budget:
        sc = nodes[v][0] + float(np.log(child_q[v][0]))
        nodes.append((sc, v, nodes[v][2] + 1, 0, True))
        v = len(nodes) - 1
        expand(v)
    taken = {(nodes[i][1], nodes[i][3]) for i in range(1, len(nodes))}

    heap = []

    def push_children(v):
        for r, q in enumerate(child_q[v]):
            if (v, r) not in taken:
                heapq.heappush(heap, (-(nodes[v][0] + float(np.log(q))), v, r))

    for v in range(len(nodes)):
        push_children(v)
    while len(nodes) - 1 < budget and heap:
        negs, p, r = heapq.heappop(heap)
        nodes.append((-negs, p, nodes[p][2] + 1, r, False))
        taken.add((p, r))
        v = len(nodes) - 1
        expand(v)
        push_children(v)

    # order the draft nodes by descending score; scores fall strictly along a
    # path so every parent precedes its children
    order = sorted(range(1, len(nodes)), key=lambda i: (-nodes[i][0], i))
    new_index = {0: -1}
    for k, i in enumerate(order):
        new_index[i] = k
    parent = np.array([new_index[nodes[i][1]] for i in order], np.int32)
    depth = np.array([nodes[i][2] for i in order], np.int32)
    main = np.array([nodes[i][4] for i in order], bool)
    for k in range(len(order)):
        assert parent[k] < k
    return parent, depth, main


def tree_drafts(S, g, budget, branching, max_depth, alpha, vocab, cfg_index,
                req, step):
    """Tokens for a best-first tree.  Main-path nodes carry the reference
    token with probability alpha; every other node is uniform over the
    vocabulary minus the reference token at its depth (so only the main path
    can be accepted and the acceptance law stays closed-form)."""
    parent, depth, main = tree_topology(budget, branching, max_depth,
                                        cfg_index, step)
    rng = np.random.default_rng([200, cfg_index, req, step])
    toks = np.empty(len(parent), np.int32)
    for k in range(len(parent)):
        tgt = _target(S, g, int(depth[k]))
        if main[k] and tgt is not None and rng.random() < alpha:
            toks[k] = tgt
        else:
            toks[k] = _not_equal(rng, vocab, tgt)
    return toks, parent


def batched_mix(n_req, ctx_lo, ctx_hi, alpha_lo, alpha_hi):
    """Per-request context length ~ U{ctx_lo..ctx_hi} and alpha ~ U(lo, hi)."""
    rng = np.random.default_rng(300)
    ctx = rng.integers(ctx_lo, ctx_hi + 1, size=n_req)
    alpha = rng.uniform(alpha_lo, alpha_hi, size=n_req)
    return ctx.astype(np.int32), alpha


def expected_tokens_per_step(alpha, K):
    """E[tokens emitted per step] when each of K chain positions matches
    independently with probability alpha (accepted prefix plus the bonus)."""
    if alpha == 1.0:
        return float(K + 1)
    return 1.0 + alpha * (1.0 - alpha ** K) / (1.0 - alpha)
