"""Pins of the oracle's building blocks against closed forms and library
routines (bf16 rounding, RMSNorm, RoPE, masked softmax attention, the
recurrence)."""

import math

import numpy as np
import pytest
import torch

from oracle import (bf16_round, rmsnorm, rope_tables, apply_rope,
                    masked_attention, sigmoid, silu, Model)


# ---------------------------------------------------------------- bf16 (P6)

def test_bf16_round_matches_torch_random():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(500_000).astype(np.float32),
        (rng.standard_normal(250_000) * 1e30).astype(np.float32),
        (rng.standard_normal(250_000) * 1e-39).astype(np.float32),  # subnormal
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    got = bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_bf16_round_boundaries():
    bits = np.array([
        0x3F808000,  # exact tie, even below -> stays 0x3F80
        0x3F818000,  # exact tie, odd below  -> rounds up to 0x3F82
        0x3F808001,  # just above the tie    -> up
        0x3F807FFF,  # just below the tie    -> down
        0x7F7FFFFF,  # FLT_MAX               -> rounds to +inf
        0xFF7FFFFF,  # -FLT_MAX              -> -inf
        0x00000001,  # smallest subnormal    -> 0
        0x80000000,  # -0
        0x7F800000,  # +inf
        0x00408000,  # subnormal tie
    ], dtype=np.uint32)
    x = bits.view(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).float().numpy()
    got = bf16_round(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    expect_hi = [0x3F80, 0x3F82, 0x3F81, 0x3F80, 0x7F80, 0xFF80, 0x0000,
                 0x8000, 0x7F80, 0x0040]
    assert list(got.view(np.uint32) >> 16) == expect_hi
    assert np.isnan(bf16_round(np.array([np.nan], np.float32)))[0]


# ------------------------------------------------------------- RMSNorm (P5)

@pytest.mark.parametrize("c", [3.0, -0.5, 1e-3, 7.25])
def test_rmsnorm_constant_vector_closed_form(c):
    eps = 1e-6
    x = np.full((1, 64), c, np.float32)
    got = rmsnorm(x, np.ones(64, np.float32), eps)
    expect = math.copysign(1.0, c) / math.sqrt(1.0 + eps / (c * c))
    assert np.allclose(got, expect, rtol=1e-6, atol=0)


def test_rmsnorm_unit_rms_and_weight():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 256)).astype(np.float32) * 3
    w = rng.standard_normal(256).astype(np.float32)
    y = rmsnorm(x, np.ones(256, np.float32), 0.0)
    assert np.allclose(np.sqrt(np.mean(y.astype(np.float64) ** 2, axis=1)), 1.0,
                       atol=1e-6)
    assert np.allclose(rmsnorm(x, w, 0.0), y * w, rtol=1e-6, atol=1e-7)


# ---------------------------------------------------------------- RoPE (P5)

def test_rope_position_zero_is_identity_and_norm_preserving():
    cos, sin = rope_tables(64, 32, 10000.0)
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 3, 32)).astype(np.float32)
    y0 = apply_rope(x, np.zeros(6, np.int64), cos, sin)
    assert np.array_equal(y0, x)
    y = apply_rope(x, np.arange(6) * 7, cos, sin)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1),
                       rtol=1e-5)


def test_rope_scores_depend_only_on_relative_position():
    """<RoPE(q, m), RoPE(k, n)> is a function of m - n: a wrong pairing of
    the rotated halves or a sign slip breaks it."""
    cos, sin = rope_tables(512, 64, 10000.0)
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 64)).astype(np.float32)
    k = rng.standard_normal((1, 1, 64)).astype(np.float32)

    def score(m, n):
        a = apply_rope(q, np.array([m]), cos, sin)
        b = apply_rope(k, np.array([n]), cos, sin)
        return float(np.sum(a.astype(np.float64) * b))
    for delta in (0, 1, 5, 40):
        ref = score(100 + delta, 100)
        for base in (0, 17, 300):
            assert abs(score(base + delta, base) - ref) < 2e-4


def test_rope_table_values():
    cos, sin = rope_tables(8, 4, 10000.0)
    # hd = 4: inv_freq = [1, 10000^-0.5]
    assert abs(float(cos[3, 0]) - math.cos(3.0)) < 1e-7
    assert abs(float(sin[5, 1]) - math.sin(5.0 * 0.01)) < 1e-7


# ----------------------------------------------------------- attention (P5)

def test_attention_single_allowed_key_returns_its_value():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((3, 4, 16)).astype(np.float32)
    keys = rng.standard_normal((10, 2, 16)).astype(np.float32)
    vals = rng.standard_normal((10, 2, 16)).astype(np.float32)
    allowed = np.zeros((3, 10), bool)
    allowed[0, 7] = allowed[1, 0] = allowed[2, 9] = True
    o = masked_attention(q, keys, vals, allowed, 0.25)
    for r, j in ((0, 7), (1, 0), (2, 9)):
        for h in range(4):
            assert np.allclose(o[r, h], vals[j, h // 2])


def test_attention_equal_scores_give_mean_and_weights_sum_to_one():
    rng = np.random.default_rng(5)
    q = np.zeros((2, 2, 8), np.float32)
    keys = rng.standard_normal((6, 1, 8)).astype(np.float32)
    vals = rng.standard_normal((6, 1, 8)).astype(np.float32)
    allowed = np.array([[1, 1, 0, 1, 0, 0], [1, 1, 1, 1, 1, 1]], bool)
    o = masked_attention(q, keys, vals, allowed, 1.0)
    assert np.allclose(o[0, 0], vals[[0, 1, 3], 0].mean(0), atol=1e-6)
    assert np.allclose(o[1, 1], vals[:, 0].mean(0), atol=1e-6)
    ones = np.ones((6, 1, 8), np.float32)
    q2 = rng.standard_normal((2, 2, 8)).astype(np.float32)
    assert np.allclose(masked_attention(q2, keys, ones, allowed, 0.3), 1.0,
                       atol=1e-6)


def test_attention_matches_float64_softmax():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, 4, 16)).astype(np.float32)
    keys = rng.standard_normal((9, 2, 16)).astype(np.float32)
    vals = rng.standard_normal((9, 2, 16)).astype(np.float32)
    allowed = rng.random((4, 9)) < 0.6
    allowed[:, 0] = True
    o = masked_attention(q, keys, vals, allowed, 0.25)
    for r in range(4):
        for h in range(4):
            idx = np.nonzero(allowed[r])[0]
            s = keys[idx, h // 2].astype(np.float64) @ q[r, h] * 0.25
            p = np.exp(s - s.max())
            p /= p.sum()
            assert np.allclose(o[r, h], p @ vals[idx, h // 2], atol=1e-6)


# ---------------------------------------------------------- recurrence (P4)

def _rec_inputs(R, d, S, seed):
    rng = np.random.default_rng(seed)
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return f(d, S), f(R, d), f(R, d), f(R, d), f(R, S), f(R, S)


def test_recurrence_gate_open_sums_inputs():
    """sigmoid(a) = 1: H_t = H_0 + sum_{u<=t} B_u x_u."""
    R, d, S = 5, 6, 4
    H0, x, _, z, B, C = _rec_inputs(R, d, S, 8)
    a = np.full((R, d), 60.0, np.float32)
    o, Hs = Model._recurrence(H0, np.arange(-1, R - 1), x, a, z, B, C)
    H = H0.astype(np.float64)
    for t in range(R):
        H = H + np.outer(x[t], B[t])
        y = H @ C[t]
        assert np.allclose(o[t], y * silu(z[t]), rtol=1e-5, atol=1e-5)
    assert np.allclose(Hs[R - 1], H, atol=1e-5)


def test_recurrence_gate_closed_forgets_history():
    """sigmoid(a) = 0: H_t = B_t x_t, so y_t = x_t (B_t . C_t)."""
    R, d, S = 4, 5, 3
    H0, x, _, z, B, C = _rec_inputs(R, d, S, 9)
    a = np.full((R, d), -200.0, np.float32)
    o, _ = Model._recurrence(H0, np.arange(-1, R - 1), x, a, z, B, C)
    for t in range(R):
        assert np.allclose(o[t], x[t] * float(B[t] @ C[t]) * silu(z[t]),
                           rtol=1e-5, atol=1e-6)


def test_recurrence_tree_equals_per_path_sequential():
    """A node's state in a tree equals the sequential recurrence along its
    own root path, bitwise (same op order)."""
    R, d, S = 7, 5, 4
    H0, x, a, z, B, C = _rec_inputs(R, d, S, 10)
    parents = np.array([-1, 0, 0, 1, 1, 2, 5])
    o, _ = Model._recurrence(H0, parents, x, a, z, B, C)
    for i in range(R):
        path = []
        v = i
        while v != -1:
            path.append(v)
            v = parents[v]
        path.reverse()
        sel = np.array(path)
        oc, _ = Model._recurrence(H0, np.arange(-1, len(path) - 1), x[sel],
                                  a[sel], z[sel], B[sel], C[sel])
        assert np.array_equal(oc[-1], o[i])


def test_sigmoid_silu_closed_forms():
    x = np.array([-3.0, 0.0, 2.0], np.float32)
    assert np.allclose(sigmoid(x), 1 / (1 + np.exp(-x.astype(np.float64))))
    assert np.allclose(silu(x), x / (1 + np.exp(-x.astype(np.float64))))
    assert sigmoid(np.array([0.0], np.float32))[0] == 0.5
