"""Token-forcing parity harness: the GPU verify loop against the oracle.

Protocol F (per request): the oracle's greedy sequence S and its per-step
logits and top-1/top-2 margins are the reference.  Drafts are S perturbed
with match probability alpha (chains) or best-first trees with S planted on
the main path.  After each verify every emitted token is compared with S; a
mismatch is allowed only where the oracle's margin is below NEAR_TIE, is
counted, and the step is committed only up to it with the oracle's token
forced as the next root, so one near-tie never cascades.  Logits of the root
and accepted rows are compared with the oracle's AR logits; with
`all_rows` the logits of every row (rejected branches included) are
compared with the oracle's single tree-masked pass from the same committed
state.
"""

import numpy as np

import synth
from oracle import ar_greedy, Model

NEAR_TIE = 1e-2


def logit_tol(dtype, ref_row):
    """fp32 models: 1e-4 absolute; bf16 models: 2e-2 x the row's std."""
    if dtype == "fp32":
        return 1e-4
    return 2e-2 * float(np.std(ref_row))


def make_drafts(kind, S, g, w, vocab, cfg_index, req, step, alpha=None):
    alpha = w["alpha"] if alpha is None else alpha
    if kind == "chain":
        return synth.chain_drafts(S, g, w["K"], alpha, vocab, cfg_index, req, step)
    return synth.tree_drafts(S, g, w["K"], w.get("branching", (4, 3, 2, 2, 1, 1, 1, 1)),
                             w.get("max_depth", 8), alpha, vocab, cfg_index, req, step)


class Report:
    def __init__(self):
        self.steps = 0
        self.emitted = 0
        self.near_tie_mismatch = 0
        self.max_logit_err = 0.0       # in units of the tolerance
        self.rows_checked = 0
        self.first_bad = None          # (g, got, expected, margin) if not exempt
        self.tokens = []

    def __repr__(self):
        return (f"Report(steps={self.steps}, emitted={self.emitted}, "
                f"near_tie_mismatch={self.near_tie_mismatch}, "
                f"max_logit_err/tol={self.max_logit_err:.3f}, "
                f"rows={self.rows_checked}, first_bad={self.first_bad})")


def protocol_f(engine, model_cfg, oracle_model, prompt, n_gen, w, kind,
               cfg_index=0, req=0, all_rows=False, check_logits=True,
               oracle_ref=None, stop_on_bad=True, alpha=None):
    """Run spec decoding of n_gen tokens for one request and check it.
    Returns a Report.  oracle_ref: optional precomputed (S, L, M)."""
    dtype = model_cfg["dtype"]
    V = model_cfg["vocab"]
    if oracle_ref is None:
        S, Lg, M, _ = ar_greedy(oracle_model, prompt, n_gen)
    else:
        S, Lg, M = oracle_ref
    rep = Report()
    first, lg0 = engine.prefill(req, prompt, logits=True)
    lg0 = lg0.cpu().numpy()
    _check_rows(rep, dtype, lg0[None], Lg[0][None])
    if first != S[0]:
        if M[0] < NEAR_TIE:
            rep.near_tie_mismatch += 1
            engine.force_root(req, int(S[0]))
        else:
            rep.first_bad = (0, first, int(S[0]), float(M[0]))
            return rep
    g = 1
    rep.tokens.append(int(S[0]))
    ost = None
    if all_rows:
        ost = oracle_model.new_state()
        oracle_model.prefill(ost, prompt)
        pending_oracle = []          # committed tokens not yet fed to ost
    step = 0
    while g < n_gen:
        toks, par = make_drafts(kind, S, g, w, V, cfg_index, req, step, alpha)
        paths, bonus, lg = engine.verify([req], [toks], [par], logits=True)
        path, b = paths[0], bonus[0]
        lg = lg.cpu().numpy()
        emitted = [int(toks[p]) for p in path] + [int(b)]
        # compare emitted tokens with S
        j_bad = None
        for j, t in enumerate(emitted):
            if g + j >= n_gen:
                break
            if t != int(S[g + j]):
                j_bad = j
                break
        # logits: root row -> S position g; accepted node k -> g + k + 1
        if check_logits:
            rows_idx = [0] + [p + 1 for p in path]
            upto = len(rows_idx) if j_bad is None else j_bad + 1
            ref_idx = [g + k for k in range(upto) if g + k < n_gen]
            _check_rows(rep, dtype, lg[rows_idx[:len(ref_idx)]],
                        Lg[ref_idx])
        if all_rows:
            for t in pending_oracle:
                oracle_model.decode(ost, t)
            pending_oracle = []
            root = int(S[g - 1])
            nodes = np.concatenate([[root], toks])
            npar = np.concatenate([[-1], np.asarray(par) + 1])
            ref = oracle_model.forward(ost, nodes, npar)
            _check_rows(rep, dtype, lg, ref)
        if j_bad is not None:
            pos = g + j_bad
            if M[pos] < NEAR_TIE:
                rep.near_tie_mismatch += 1
            else:
                rep.first_bad = (pos, emitted[j_bad], int(S[pos]), float(M[pos]))
                if stop_on_bad:
                    return rep
            keep = path[:j_bad] if j_bad < len(path) else path
            engine.commit([req], [keep], [int(S[pos])])
            n_new = len(keep) + 1
        else:
            engine.commit([req], [path], [int(b)])
            n_new = len(emitted)
        if all_rows and g + n_new - 1 <= n_gen:
            pending_oracle = [int(S[g - 1])] + [int(S[g + k]) for k in range(n_new - 1)]
        rep.tokens.extend(int(S[g + k]) if g + k < n_gen else -1 for k in range(n_new))
        g += n_new
        rep.emitted += n_new
        rep.steps += 1
        step += 1
    return rep


def _check_rows(rep, dtype, got, ref):
    for gr, rr in zip(got, ref):
        tol = logit_tol(dtype, rr)
        err = float(np.max(np.abs(gr.astype(np.float64) - rr)))
        rep.max_logit_err = max(rep.max_logit_err, err / tol)
        rep.rows_checked += 1


def engine_for(model_cfg, weights, **caps):
    from tree_verification_spec_amd import Engine
    e = Engine(model_cfg, **caps)
    e.load_weights([weights[name] for name, _, _ in synth.tensor_specs(model_cfg)])
    return e


def oracle_for(model_cfg, weights, max_pos=16384):
    return Model(model_cfg, weights, max_pos=max_pos)
