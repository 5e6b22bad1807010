"""Model shapes and workloads.

Model shapes follow the targets the SpecPilot pages evaluate (a dense
8B-class decoder and a ~27B hybrid whose recurrent layers sit between GQA
attention layers; besthub.dev article, "(2) Best-first Tree Verification for
Hybrid Architectures").  Constants the pages leave open (RoPE base, norm
epsilon, layer order of the hybrid) are fixed here once and used by both the
oracle and the GPU library.
"""

import copy

_DENSE8B = dict(
    n_layers=36, d_model=4096, n_heads=32, n_kv_heads=8, head_dim=128,
    ffn_dim=12288, vocab=151936, dtype="bf16", lr_state=0,
    layer_kinds="A" * 36, rms_eps=1e-6, rope_theta=10000.0, seed_w=1,
)

_HYBRID27B = dict(
    n_layers=64, d_model=5120, n_heads=40, n_kv_heads=8, head_dim=128,
    ffn_dim=17408, vocab=151936, dtype="bf16", lr_state=64,
    layer_kinds="LLLA" * 16, rms_eps=1e-6, rope_theta=10000.0, seed_w=2,
)

_TINY = dict(
    n_layers=2, d_model=256, n_heads=4, n_kv_heads=4, head_dim=64,
    ffn_dim=1024, vocab=4096, dtype="fp32", lr_state=0,
    layer_kinds="AA", rms_eps=1e-6, rope_theta=10000.0, seed_w=0,
)


def _variant(base, **kw):
    c = copy.deepcopy(base)
    c.update(kw)
    if "layer_kinds" not in kw:
        c["layer_kinds"] = base["layer_kinds"][: c["n_layers"]]
    return c


MODELS = {
    # the five workloads' models
    "tiny": _TINY,
    "dense8b": _DENSE8B,
    "hybrid27b": _HYBRID27B,
    # full-width, few-layer variants: real d, heads, FFN and vocab
    "dense8b_l2": _variant(_DENSE8B, n_layers=2),
    "hybrid27b_l4": _variant(_HYBRID27B, n_layers=4),
    # small shapes that exercise GQA, bf16 rounding and the recurrent layers
    "tiny_gqa": _variant(_TINY, n_heads=8, n_kv_heads=2, head_dim=64,
                         n_layers=2, ffn_dim=512, vocab=1024),
    "tiny_gqa_bf16": _variant(_TINY, n_heads=8, n_kv_heads=2, head_dim=64,
                              d_model=512, n_layers=2, ffn_dim=1024,
                              vocab=2048, dtype="bf16", seed_w=5),
    "tiny_hybrid": _variant(_TINY, n_layers=4, layer_kinds="LLLA",
                            n_heads=4, n_kv_heads=2, head_dim=64,
                            ffn_dim=512, vocab=1024, lr_state=16, seed_w=3),
    "tiny_hybrid_bf16": _variant(_TINY, n_layers=4, layer_kinds="LLLA",
                                 d_model=512, n_heads=8, n_kv_heads=2,
                                 head_dim=64, ffn_dim=1024, vocab=2048,
                                 lr_state=64, dtype="bf16", seed_w=4),
}

# The five measured workloads.  "K" counts draft tokens (the pending root is
# not a draft), so one request contributes K+1 rows to a verify pass.
WORKLOADS = {
    "tiny_chain": dict(index=0, model="tiny", prompt=64, draft="chain", K=4,
                       alpha=0.7, gen=128, batch=1),
    "dense8b_chain": dict(index=1, model="dense8b", prompt=2048,
                          draft="chain", K=16, alpha=0.7,
                          alphas=(0.5, 0.7, 0.9), gen=512, batch=1),
    "dense8b_tree": dict(index=2, model="dense8b", prompt=4096, draft="tree",
                         K=64, alpha=0.8, gen=512, batch=1,
                         branching=(4, 3, 2, 2, 1, 1, 1, 1), max_depth=8),
    "dense8b_batched": dict(index=3, model="dense8b", prompt=None,
                            draft="chain", K=8, alpha=None, gen=None,
                            steps=128, batch=32, ctx_lo=512, ctx_hi=4096,
                            alpha_lo=0.4, alpha_hi=0.9, page=16),
    "hybrid27b_tree": dict(index=4, model="hybrid27b", prompt=2048,
                           draft="tree", K=32, alpha=0.8, gen=512, batch=1,
                           branching=(4, 3, 2, 2, 1, 1, 1, 1), max_depth=8),
}


def model_config(name):
    c = copy.deepcopy(MODELS[name])
    c["name"] = name
    assert len(c["layer_kinds"]) == c["n_layers"]
    assert c["n_heads"] % c["n_kv_heads"] == 0
    return c


def workload(name):
    w = copy.deepcopy(WORKLOADS[name])
    w["name"] = name
    return w
