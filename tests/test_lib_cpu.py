"""Host-side checks that need no GPU: the C-ABI library loads, exports every
symbol its header declares, and sizes its workspace from a config."""

import ctypes
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from tree_verification_spec_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("libspec.so is not built (run __graft_entry__.build())")
    return L


def test_header_symbols_are_exported():
    L = _lib()
    header = open(os.path.join(ROOT, "include", "spec.h")).read()
    declared = set(re.findall(r"\b(spec_[a-z_]+)\s*\(", header))
    assert "spec_verify" in declared and "spec_commit" in declared
    so = ctypes.CDLL(L.LIB_PATH)
    for name in declared:
        assert hasattr(so, name), name
    assert declared == set(L.EXPORTS)


def test_workspace_bytes_and_config_validation():
    L = _lib()
    from tree_verification_spec_amd import make_config
    tiny = synth.model_config("tiny")
    n = L.spec_workspace_bytes(make_config(tiny, max_ctx=512, max_nodes=5))
    # the weights alone
    w = sum(int(__import__("numpy").prod(s)) for _, s, _ in synth.tensor_specs(tiny)) * 4
    assert n > w
    big = synth.model_config("dense8b")
    n8 = L.spec_workspace_bytes(make_config(big, max_ctx=2600, max_nodes=17))
    assert 16.3e9 < n8 < 20e9
    bad = make_config(tiny, max_nodes=66)
    assert L.spec_workspace_bytes(bad) == 0
    odd = dict(tiny, head_dim=96)
    assert L.spec_workspace_bytes(make_config(odd)) == 0
    # model width: a multiple of 32 up to 16384 (the row kernels' register tiles)
    assert L.spec_workspace_bytes(make_config(dict(tiny, d_model=48))) == 0
    wide = dict(tiny, d_model=16384 + 32)
    assert L.spec_workspace_bytes(make_config(wide)) == 0
    # W12 weight storage: bf16 models only
    assert L.spec_workspace_bytes(make_config(tiny, weight_format="w12")) == 0
    b16 = synth.model_config("tiny_gqa_bf16")
    assert L.spec_workspace_bytes(make_config(b16, weight_format="w12")) > 0
    # W12 plus the 8-bit view: bf16 only, one more byte per weight
    assert L.spec_workspace_bytes(make_config(tiny, weight_format="w12_lowp")) == 0
    w12 = L.spec_workspace_bytes(make_config(b16, weight_format="w12"))
    lowp = L.spec_workspace_bytes(make_config(b16, weight_format="w12_lowp"))
    n_w = sum(int(np.prod(s)) for n, s, k in synth.tensor_specs(b16)
              if k == "mat" and n != "embed")
    assert lowp - w12 >= n_w
    bad_fmt = make_config(b16)
    bad_fmt.weight_format = 3
    assert L.spec_workspace_bytes(bad_fmt) == 0
    # the attention split table covers 64 splits of 128 keys
    assert L.spec_workspace_bytes(make_config(tiny, max_ctx=8192)) > 0
    assert L.spec_workspace_bytes(make_config(tiny, max_ctx=8193)) == 0


def test_product_path_has_no_oracle_dependency():
    """The library package must not import the oracle."""
    pkg = os.path.join(ROOT, "tree_verification_spec_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle", text, re.M), f
                assert "oracle/" not in text, f


def test_kv_pool_size_follows_kv_pages():
    """The KV pool is kv_pages pages of 16 tokens (K and V of every attention
    layer); 0 sizes it for every request at max_ctx; negative is invalid."""
    L = _lib()
    from tree_verification_spec_amd import make_config
    tiny = synth.model_config("tiny")
    full = L.spec_workspace_bytes(make_config(tiny, max_requests=4, max_ctx=512, max_nodes=5))
    default_pages = 4 * 512 // 16
    small = L.spec_workspace_bytes(make_config(tiny, max_requests=4, max_ctx=512, max_nodes=5,
                                               kv_pages=40))
    n_attn = tiny["layer_kinds"].count("A")
    per_page = 2 * n_attn * tiny["n_kv_heads"] * 16 * tiny["head_dim"] * 4
    assert abs((full - small) - (default_pages - 40) * per_page) <= 4096
    assert L.spec_workspace_bytes(make_config(tiny, kv_pages=-1)) == 0

