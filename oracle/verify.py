"""Greedy tree verification, acceptance and AR decoding for the oracle.
TEST INFRASTRUCTURE.

Acceptance (besthub.dev article, "(2) Best-first Tree Verification for Hybrid
Architectures" and "(3) Two-Level Verification": only the exact verification
accepts tokens; zicq.com article, "Core Idea": every emitted token must equal
the stock greedy output):

    A(i)  = argmax_v logits(i)[v]         (lowest v among equal maxima)
    ok(0) = true
    ok(i) = ok(parent(i)) and token(i) == A(parent(i))
    best  = the deepest node with ok (lowest index among equally deep ones)
    path  = the draft nodes from the root down to best; bonus = A(best)

The tokens emitted by a step are the path's tokens followed by the bonus.
"""

import numpy as np

from .model import tree_layout


def argmax_lowest(logits):
    """Index of the maximum; numpy returns the first (lowest) index on ties."""
    return int(np.argmax(logits))


def top2_margin(logits):
    """top1 - top2 over two distinct indices."""
    part = np.partition(np.asarray(logits, np.float32), -2)
    return float(part[-1] - part[-2])


def accept_path(node_tokens, parents, A):
    """node_tokens/parents/A over all R nodes (node 0 is the root).
    Returns (path, bonus) with path = accepted node indices (root excluded)
    in root-to-leaf order."""
    R = len(node_tokens)
    depth, _ = tree_layout(parents)
    ok = np.zeros(R, bool)
    ok[0] = True
    for i in range(1, R):
        p = int(parents[i])
        ok[i] = ok[p] and int(node_tokens[i]) == int(A[p])
    best = 0
    for i in range(R):
        if ok[i] and depth[i] > depth[best]:
            best = i
    path = []
    v = best
    while v != 0:
        path.append(v)
        v = int(parents[v])
    path.reverse()
    return path, int(A[best])


def _nodes(root, drafts, draft_parents):
    """Node arrays from the draft arrays (draft parent -1 = the root)."""
    toks = np.concatenate([[root], np.asarray(drafts, np.int64)])
    par = np.concatenate([[-1], np.asarray(draft_parents, np.int64) + 1])
    par[0] = -1
    return toks, par


def verify_single_pass(model, state, root, drafts, draft_parents):
    """One tree-masked pass over root + drafts.  Returns
    (logits[R, V], A[R], path (draft indices, 0-based), bonus)."""
    toks, par = _nodes(root, drafts, draft_parents)
    logits = model.forward(state, toks, par)
    A = np.array([argmax_lowest(r) for r in logits])
    path, bonus = accept_path(toks, par, A)
    return logits, A, [p - 1 for p in path], bonus


def verify_bruteforce(model, state, root, drafts, draft_parents):
    """Per-node logits by feeding each node's root path token by token from
    a copy of the committed state (no tree mask involved)."""
    toks, par = _nodes(root, drafts, draft_parents)
    R = len(toks)
    out = np.zeros((R, model.cfg["vocab"]), np.float32)
    for i in range(R):
        chain = []
        v = i
        while v != -1:
            chain.append(int(toks[v]))
            v = int(par[v])
        chain.reverse()
        st = state.copy()
        lg = None
        for t in chain:
            lg = model.decode(st, t)
        out[i] = lg
    A = np.array([argmax_lowest(r) for r in out])
    path, bonus = accept_path(toks, par, A)
    return out, A, [p - 1 for p in path], bonus


def ar_greedy(model, prompt, n_gen, state=None, log=None):
    """Plain autoregressive greedy decoding.  Returns
    (S[n_gen], logits[n_gen, V], margins[n_gen], state): S[0] is the argmax
    of the last prompt row, S[t+1] the argmax after feeding S[t]."""
    st = state if state is not None else model.new_state()
    lg = model.prefill(st, prompt)
    S, L, M = [], [], []
    for t in range(n_gen):
        L.append(lg)
        M.append(top2_margin(lg))
        S.append(argmax_lowest(lg))
        if log is not None:
            log(t)
        if t + 1 < n_gen:
            lg = model.decode(st, S[-1])
    return (np.array(S, np.int32), np.array(L, np.float32),
            np.array(M, np.float32), st)
