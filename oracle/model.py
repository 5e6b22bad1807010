"""Plain fp32 target model for the oracle (numpy, CPU).  TEST INFRASTRUCTURE.

Dense layers: pre-norm decoder, fp32 residual stream ``h``::

    u = rmsnorm(h) * w_attn_norm
    q, k, v = u Wq^T, u Wk^T, u Wv^T ; RoPE(q, k) at each row's position
    o = softmax(q k^T / sqrt(hd) over the allowed keys) v   (GQA: query head
        j reads kv head j // (n_heads / n_kv_heads))
    h += o Wo^T
    u = rmsnorm(h) * w_ffn_norm ; h += (silu(u Wg^T) * (u Wu^T)) Wd^T
    logits = (rmsnorm(h) * w_final) W_lm^T

Recurrent (hybrid) layers replace the attention half with a gated diagonal
linear recurrence per channel c and state index s::

    [x | a | z | B | C] = u W_in^T
    H_t[c, s] = sigmoid(a_t[c]) H_{t-1}[c, s] + B_t[s] x_t[c]
    y_t[c] = sum_s H_t[c, s] C_t[s] ;  h += (y_t * silu(z_t)) W_out^T

For a draft tree the state of a node comes from running the recurrence along
its own root path, from the committed state, so that sibling branches never
see each other's updates (besthub.dev article, section "(2) Best-first Tree
Verification for Hybrid Architectures").

Precision: fp32 models are fp32 throughout.  bf16 models hold bf16 weight
values and a bf16 KV cache: k (after RoPE) and v are rounded to bf16
(round-to-nearest-even) when they are written to the cache.  Everything else
(activations, queries, scores, softmax weights, the recurrent state) is fp32.
"""

import math
from dataclasses import dataclass, field

import numpy as np

F32 = np.float32


# ---------------------------------------------------------------- primitives

def bf16_round(x):
    """Round float32 values to the nearest bf16 value (ties to even),
    returned as float32.  NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=F32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = r.view(F32).reshape(x.shape)
    return np.where(np.isnan(x), x, out)


def rmsnorm(x, w, eps):
    """x / sqrt(mean(x^2) + eps) * w, over the last axis."""
    x = np.asarray(x, F32)
    ms = np.mean(x * x, axis=-1, keepdims=True, dtype=F32)
    return (x / np.sqrt(ms + F32(eps))) * w


def sigmoid(x):
    return F32(1) / (F32(1) + np.exp(-np.asarray(x, F32)))


def silu(x):
    x = np.asarray(x, F32)
    return x / (F32(1) + np.exp(-x))


def rope_tables(max_pos, head_dim, theta):
    """cos/sin tables [max_pos, head_dim/2]: angle = p * theta^(-2i/hd),
    evaluated in float64 and rounded once to float32."""
    half = head_dim // 2
    inv = np.array([theta ** (-2.0 * i / head_dim) for i in range(half)],
                   dtype=np.float64)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(F32), np.sin(ang).astype(F32)


def apply_rope(x, pos, cos, sin):
    """Rotate-half RoPE: pairs (i, i + hd/2) rotate by the angle of
    position pos.  x: [R, heads, hd]; pos: [R]."""
    half = x.shape[-1] // 2
    c = cos[pos][:, None, :]
    s = sin[pos][:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1).astype(F32)


def masked_attention(q, keys, vals, allowed, scale):
    """q: [R, nq, hd]; keys/vals: [L, nkv, hd]; allowed: [R, L] bool.
    Softmax attention per query head over the allowed keys."""
    R, nq, hd = q.shape
    nkv = keys.shape[1]
    group = nq // nkv
    out = np.zeros((R, nq, hd), F32)
    for j in range(nq):
        kh = j // group
        s = (q[:, j, :] @ keys[:, kh, :].T) * F32(scale)          # [R, L]
        s = np.where(allowed, s, -np.inf).astype(F32)
        m = np.max(s, axis=1, keepdims=True)
        p = np.exp(s - m)
        p = p / np.sum(p, axis=1, keepdims=True, dtype=F32)
        out[:, j, :] = p @ vals[:, kh, :]
    return out


def tree_layout(parents):
    """parents: [R] with parents[0] == -1 (node 0 is the root) and
    parents[i] < i.  Returns (depth[R], anc[R, R]) where anc[i, j] says node j
    is node i or one of its ancestors."""
    parents = np.asarray(parents)
    R = len(parents)
    depth = np.zeros(R, np.int64)
    anc = np.zeros((R, R), bool)
    for i in range(R):
        p = int(parents[i])
        if i == 0:
            assert p == -1
        else:
            assert 0 <= p < i, "parents must be topological"
            depth[i] = depth[p] + 1
            anc[i] = anc[p]
        anc[i, i] = True
    return depth, anc


# --------------------------------------------------------------------- model

@dataclass
class State:
    """Committed context of one request: KV of every attention layer for
    positions [0, n) and the recurrent state of every recurrent layer."""
    n: int = 0
    k: list = field(default_factory=list)   # per attention layer [n, nkv, hd]
    v: list = field(default_factory=list)
    H: list = field(default_factory=list)   # per recurrent layer [d, S]

    def copy(self):
        return State(self.n, [a.copy() for a in self.k],
                     [a.copy() for a in self.v], [a.copy() for a in self.H])


class Model:
    def __init__(self, cfg, weights, max_pos=16384):
        self.cfg = cfg
        self.w_raw = weights
        self._w = {}
        self.bf16 = cfg["dtype"] == "bf16"
        # storage rounding of the KV cache (identity for fp32 models)
        self.kv_rnd = bf16_round if self.bf16 else (lambda a: np.asarray(a, F32))
        self.cos, self.sin = rope_tables(max_pos, cfg["head_dim"],
                                         cfg["rope_theta"])
        self.scale = F32(1.0 / math.sqrt(cfg["head_dim"]))
        self.eps = cfg["rms_eps"]

    def W(self, name):
        """float32 view of a weight (bf16 bit patterns are widened once)."""
        if name not in self._w:
            a = self.w_raw[name]
            if a.dtype == np.uint16:
                a = (a.astype(np.uint32) << 16).view(F32)
            self._w[name] = np.asarray(a, F32)
        return self._w[name]

    def new_state(self):
        c = self.cfg
        st = State()
        for kind in c["layer_kinds"]:
            if kind == "A":
                st.k.append(np.zeros((0, c["n_kv_heads"], c["head_dim"]), F32))
                st.v.append(np.zeros((0, c["n_kv_heads"], c["head_dim"]), F32))
            else:
                st.H.append(np.zeros((c["d_model"], c["lr_state"]), F32))
        return st

    # -- one pass over a token tree ---------------------------------------
    def forward(self, state, tokens, parents, want_kv=False):
        """Score every node of a token tree in one pass.

        tokens[R], parents[R] (parents[0] == -1).  Node i sits at position
        state.n + depth(i) and attends to the committed keys [0, n) plus its
        own root path.  The committed state is not modified.  Returns
        logits [R, vocab] (and, with want_kv, the per-layer node K/V and the
        per-layer node recurrent states of the last node of each chain link).
        """
        c, kv_rnd = self.cfg, self.kv_rnd
        tokens = np.asarray(tokens, np.int64)
        R = len(tokens)
        n = state.n
        depth, anc = tree_layout(parents)
        pos = n + depth
        allowed = np.concatenate([np.ones((R, n), bool), anc], axis=1)
        nq, nkv, hd = c["n_heads"], c["n_kv_heads"], c["head_dim"]
        d, S = c["d_model"], c["lr_state"]

        h = self.W("embed")[tokens].astype(F32)
        new_k, new_v, last_H = [], [], []
        ia = il = 0
        for li, kind in enumerate(c["layer_kinds"]):
            p = f"layers.{li}."
            u = rmsnorm(h, self.W(p + "attn_norm"), self.eps)
            if kind == "A":
                q = (u @ self.W(p + "wq").T).reshape(R, nq, hd)
                k = (u @ self.W(p + "wk").T).reshape(R, nkv, hd)
                v = (u @ self.W(p + "wv").T).reshape(R, nkv, hd)
                q = apply_rope(q, pos, self.cos, self.sin)
                k = kv_rnd(apply_rope(k, pos, self.cos, self.sin))
                v = kv_rnd(v)
                keys = np.concatenate([state.k[ia], k], axis=0)
                vals = np.concatenate([state.v[ia], v], axis=0)
                o = masked_attention(q, keys, vals, allowed, self.scale)
                o = o.reshape(R, nq * hd)
                h = h + o @ self.W(p + "wo").T
                new_k.append(k)
                new_v.append(v)
                ia += 1
            else:
                proj = u @ self.W(p + "w_in").T
                x, a, z = proj[:, :d], proj[:, d:2 * d], proj[:, 2 * d:3 * d]
                Bm, Cm = proj[:, 3 * d:3 * d + S], proj[:, 3 * d + S:]
                o, Hs = self._recurrence(state.H[il], parents, x, a, z, Bm, Cm)
                h = h + o @ self.W(p + "w_out").T
                last_H.append(Hs)
                il += 1
            u = rmsnorm(h, self.W(p + "ffn_norm"), self.eps)
            g = u @ self.W(p + "wg").T
            up = u @ self.W(p + "wu").T
            act = silu(g) * up
            h = h + act @ self.W(p + "wd").T
        u = rmsnorm(h, self.W("final_norm"), self.eps)
        logits = (u @ self.W("lm_head").T).astype(F32)
        if want_kv:
            return logits, (new_k, new_v, last_H, pos)
        return logits

    @staticmethod
    def _recurrence(H0, parents, x, a, z, Bm, Cm):
        """Per-node state along each root path; returns (o[R, d], states)
        where states maps node -> H for the nodes still referenced at the
        end (the leaves).  Op order: t1 = sigmoid(a) H, t2 = B x, H = t1 + t2."""
        R, d = x.shape
        parents = np.asarray(parents)
        last_child = np.full(R, -1)
        for i in range(1, R):
            last_child[parents[i]] = i
        H = {}
        o = np.zeros((R, d), F32)
        sa = sigmoid(a)
        for i in range(R):
            pi = int(parents[i])
            Hp = H0 if pi < 0 else H[pi]
            t1 = sa[i][:, None] * Hp
            t2 = x[i][:, None] * Bm[i][None, :]
            Hi = (t1 + t2).astype(F32)
            y = Hi @ Cm[i]
            o[i] = y * silu(z[i])
            H[i] = Hi
            if pi >= 0 and last_child[pi] == i:
                del H[pi]            # no later child needs the parent state
        return o, H

    # -- committed-state updates ------------------------------------------
    def append(self, state, tokens):
        """Feed a chain of tokens: returns their logits and advances the
        committed state (KV appended, recurrent state carried forward)."""
        tokens = np.asarray(tokens, np.int64)
        R = len(tokens)
        parents = np.arange(-1, R - 1)
        logits, (nk, nv, lastH, pos) = self.forward(state, tokens, parents,
                                                    want_kv=True)
        for i in range(len(nk)):
            state.k[i] = np.concatenate([state.k[i], nk[i]], axis=0)
            state.v[i] = np.concatenate([state.v[i], nv[i]], axis=0)
        for i in range(len(lastH)):
            state.H[i] = lastH[i][R - 1]
        state.n += R
        return logits

    def prefill(self, state, prompt, chunk=1024):
        """Process the prompt; returns the logits of its last row."""
        prompt = np.asarray(prompt)
        logits = None
        for s in range(0, len(prompt), chunk):
            logits = self.append(state, prompt[s:s + chunk])
        return logits[-1]

    def decode(self, state, token):
        """One autoregressive step: feed `token`, return its logits."""
        return self.append(state, [token])[0]
