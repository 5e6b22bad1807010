"""The token-forcing checker itself, run on the CPU against an engine backed
by the oracle (no GPU): it must pass an exact implementation and flag an
injected logit bias exactly at the first generated token it affects (the
fault-injection idea of the besthub.dev article, "Phase 4: Final
Validation")."""

import numpy as np

import synth
from oracle import Model, ar_greedy, verify_single_pass
from parity import protocol_f


class OracleEngine:
    """Same calls as the GPU Engine, computed by the oracle."""

    def __init__(self, model, bias=None):
        self.m = model
        self.bias = bias      # (token, value, after_position) or None
        self.st = {}
        self.root = {}
        self.last = None

    def _biased(self, logits, positions):
        if self.bias is None:
            return logits
        tok, val, after = self.bias
        logits = logits.copy()
        for r, p in enumerate(positions):
            if p >= after:
                logits[r, tok] += val
        return logits

    def prefill(self, req, prompt, logits=False):
        st = self.m.new_state()
        lg = self.m.prefill(st, prompt)
        lg = self._biased(lg[None], [len(prompt) - 1])[0]
        self.st[req] = st
        self.root[req] = int(np.argmax(lg))
        return (self.root[req], _T(lg)) if logits else self.root[req]

    def force_root(self, req, tok):
        self.root[req] = tok

    def verify(self, reqs, drafts, parents, logits=False):
        (r,), (toks,), (par,) = reqs, drafts, parents
        st = self.st[r]
        nodes = np.concatenate([[self.root[r]], toks]).astype(np.int64)
        npar = np.concatenate([[-1], np.asarray(par) + 1])
        lg = self.m.forward(st, nodes, npar)
        depth = np.zeros(len(nodes), int)
        for i in range(1, len(nodes)):
            depth[i] = depth[npar[i]] + 1
        lg = self._biased(lg, st.n + depth)
        A = np.argmax(lg, axis=1)
        from oracle import accept_path
        path, bonus = accept_path(nodes, npar, A)
        self.last = (r, nodes)
        out = ([[p - 1 for p in path]], [bonus])
        return out + (_T(lg),) if logits else out

    def commit(self, reqs, paths, roots):
        r, nodes = self.last
        seq = [int(nodes[0])] + [int(nodes[p + 1]) for p in paths[0]]
        for t in seq:
            self.m.decode(self.st[r], t)
        self.root[r] = int(roots[0])


class _T:
    def __init__(self, a):
        self.a = a

    def cpu(self):
        return self

    def numpy(self):
        return self.a

    def __getitem__(self, i):
        return _T(self.a[i])


def _setup():
    cfg = synth.model_config("tiny_gqa")
    w = synth.make_weights(cfg)
    return cfg, Model(cfg, w, max_pos=1024)


def test_checker_passes_exact_engine():
    cfg, m = _setup()
    w = dict(K=5, alpha=0.7, branching=(4, 3, 2, 2, 1, 1, 1, 1), max_depth=8)
    prompt = synth.prompt_tokens(cfg["vocab"], 30, 70)
    for kind in ("chain", "tree"):
        rep = protocol_f(OracleEngine(m), cfg, m, prompt, 30, w, kind,
                         cfg_index=70, all_rows=True)
        assert rep.first_bad is None and rep.near_tie_mismatch == 0, rep
        assert rep.max_logit_err < 0.05, rep
        assert rep.emitted + 1 >= 30


def test_checker_flags_late_logit_bias_at_first_affected_token():
    cfg, m = _setup()
    w = dict(K=5, alpha=0.7)
    prompt = synth.prompt_tokens(cfg["vocab"], 30, 71)
    S, L, M, _ = ar_greedy(m, prompt, 60)
    after = 30 + 40
    t_star = after - 30 + 1        # the row at position `after` predicts S[t*]
    bad = int((S[t_star] + 1) % cfg["vocab"])
    rep = protocol_f(OracleEngine(m, bias=(bad, 100.0, after)), cfg, m, prompt,
                     60, w, "chain", cfg_index=71, oracle_ref=(S, L, M),
                     check_logits=False)
    assert rep.first_bad is not None
    assert rep.first_bad[0] == t_star and rep.first_bad[1] == bad
    # a bias that switches on only after the checked length is never seen
    rep2 = protocol_f(OracleEngine(m, bias=(bad, 100.0, 30 + 200)), cfg, m,
                      prompt, 60, w, "chain", cfg_index=71,
                      oracle_ref=(S, L, M), check_logits=False)
    assert rep2.first_bad is None
