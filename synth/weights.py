"""Seeded random-init weights.

Every matrix is N(0, 0.02), drawn in float32 from
``numpy.random.default_rng([seed_w, tensor_id, chunk])`` in chunks of 2**24
elements (so that generation runs on all host cores and stays reproducible),
then rounded to bf16 (round-to-nearest-even, via torch's conversion) for the
bf16 models.  Norm weights are all ones and draw nothing.

Tensor order (tensor_id): embedding; per layer either
``attn_norm, wq, wk, wv, wo, ffn_norm, wg, wu, wd`` (attention layer) or
``attn_norm, w_in, w_out, ffn_norm, wg, wu, wd`` (recurrent layer); then
``final_norm, lm_head``.  Matrices are row-major ``[out, in]``.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 24
STD = 0.02


def tensor_specs(cfg):
    """Ordered list of (name, shape, kind) with kind in {'mat', 'norm'}."""
    d, hd = cfg["d_model"], cfg["head_dim"]
    nq, nkv, f, V = cfg["n_heads"], cfg["n_kv_heads"], cfg["ffn_dim"], cfg["vocab"]
    S = cfg["lr_state"]
    specs = [("embed", (V, d), "mat")]
    for i, kind in enumerate(cfg["layer_kinds"]):
        p = f"layers.{i}."
        specs.append((p + "attn_norm", (d,), "norm"))
        if kind == "A":
            specs += [(p + "wq", (nq * hd, d), "mat"),
                      (p + "wk", (nkv * hd, d), "mat"),
                      (p + "wv", (nkv * hd, d), "mat"),
                      (p + "wo", (d, nq * hd), "mat")]
        else:
            specs += [(p + "w_in", (3 * d + 2 * S, d), "mat"),
                      (p + "w_out", (d, d), "mat")]
        specs += [(p + "ffn_norm", (d,), "norm"),
                  (p + "wg", (f, d), "mat"),
                  (p + "wu", (f, d), "mat"),
                  (p + "wd", (d, f), "mat")]
    specs += [("final_norm", (d,), "norm"), ("lm_head", (V, d), "mat")]
    return specs


def _f32_to_bf16_bits(x):
    import torch  # conversion only (round-to-nearest-even)
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits):
    """Widen bf16 bit patterns (uint16) to the float32 values they denote."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_weights(cfg, threads=None, names=None):
    """Return {name: array}.  fp32 models give float32 arrays; bf16 models
    give uint16 arrays holding bf16 bit patterns."""
    threads = threads or min(32, len(os.sched_getaffinity(0)))
    bf16 = cfg["dtype"] == "bf16"
    out, jobs = {}, []
    for tid, (name, shape, kind) in enumerate(tensor_specs(cfg)):
        if names is not None and name not in names:
            continue
        if kind == "norm":
            out[name] = (np.full(shape, 0x3F80, np.uint16) if bf16
                         else np.ones(shape, np.float32))
            continue
        arr = np.empty(shape, np.uint16 if bf16 else np.float32)
        out[name] = arr
        n = arr.size
        for c in range((n + CHUNK - 1) // CHUNK):
            jobs.append((arr.reshape(-1), tid, c, min(CHUNK, n - c * CHUNK)))

    seed_w = cfg["seed_w"]

    def run(job):
        flat, tid, c, m = job
        rng = np.random.default_rng([seed_w, tid, c])
        x = rng.standard_normal(m, dtype=np.float32)
        x *= np.float32(STD)
        flat[c * CHUNK: c * CHUNK + m] = _f32_to_bf16_bits(x) if bf16 else x

    if threads > 1 and len(jobs) > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(run, jobs))
    else:
        for j in jobs:
            run(j)
    return out
