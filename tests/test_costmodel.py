"""Cost-model report: kernel classification, lower bounds, factor identities
and trace splitting (CPU only)."""

import glob
import os
import re

import pytest

import synth
from tree_verification_spec_amd import costmodel

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NOT_IN_STEP = {"relayout_kernel", "to_f32_kernel", "w12_rowexp_kernel", "w12_encode_kernel",
               "stream_read_kernel", "xor_reduce_kernel"}


def _kernel_names():
    names = set()
    for f in glob.glob(os.path.join(ROOT, "tree_verification_spec_amd", "csrc", "*.hip")):
        src = open(f).read()
        names |= set(re.findall(r"__global__[^;{]*?\bvoid\s+(\w+)\s*\(", src, re.S))
    return names


def test_every_kernel_is_classified():
    names = _kernel_names()
    assert "gemm_kernel" in names and "attn_kernel" in names
    for n in names:
        t = costmodel.kernel_type(f"void (anonymous namespace)::{n}<unsigned short>(Args)")
        if n in NOT_IN_STEP:
            assert t is None, n
        else:
            assert t in costmodel.TYPES, n


def test_lower_bound_is_the_larger_term():
    # 90% of 8 TB/s is 7.2e12 bytes/s; 60% of 2.5 PFLOP/s is 1.5e15 FLOP/s
    assert costmodel.lower_bound(7.2e12, 0.0) == pytest.approx(1.0)
    assert costmodel.lower_bound(0.0, 1.5e15) == pytest.approx(1.0)
    assert costmodel.lower_bound(7.2e12, 3.0e15) == pytest.approx(2.0)
    assert costmodel.lower_bound(14.4e12, 1.5e15) == pytest.approx(2.0)


def test_factor_identity():
    m = {"gemm": 2600.0, "attention": 600.0, "recurrent": 0.0, "other": 700.0}
    b = {"gemm": 1600.0, "attention": 40.0, "recurrent": 0.0, "other": 0.0}
    f = costmodel.factors(m, b, 4300.0)
    assert f["profiled_us"] == 3900.0 and f["bound_us"] == 1640.0
    assert f["kernel_factor"] * f["overhead_factor"] == pytest.approx(f["total_factor"])
    assert f["total_factor"] == pytest.approx(4300.0 / 1640.0)


def test_type_bytes_match_closed_form_8b():
    """The 8B dense model's bytes per step written out: weights (36 layers of
    QKV, O, gate, up, down plus the LM head) and the KV of 2048 committed
    tokens plus 17 new rows; no recurrent state."""
    cfg = synth.model_config("dense8b")
    d, f, V = 4096, 12288, 151936
    per_layer = d * (32 * 128 + 2 * 8 * 128) + 32 * 128 * d + 3 * d * f
    params = 36 * per_layer + V * d
    kv = (2048 + 17) * 36 * 8 * 128 * 2 * 2
    tb = costmodel.type_bounds(synth.tensor_specs(cfg), cfg, [17], [2048], "native")
    assert tb["gemm"][0] == 2 * params
    assert tb["gemm"][1] == 2 * params * 17
    assert tb["attention"][0] == kv
    assert tb["recurrent"] == (0.0, 0.0) and tb["other"] == (0.0, 0.0)
    rows = 36 * (32 * 128 + 2 * 8 * 128 + d + 2 * f + d) + V
    tw = costmodel.type_bounds(synth.tensor_specs(cfg), cfg, [17], [2048], "w12")
    assert tw["gemm"][0] == pytest.approx(params * 800 / 512 + rows)


def test_hybrid_state_bytes():
    cfg = synth.model_config("hybrid27b")
    n_lr = cfg["layer_kinds"].count("L")
    tb = costmodel.type_bounds(synth.tensor_specs(cfg), cfg, [33, 33], [100, 200], "native")
    assert tb["recurrent"][0] == 2 * 2 * n_lr * cfg["d_model"] * cfg["lr_state"] * 4


def _row(name, t0, dt, grid_x=64):
    return {"Kernel_Name": name, "Start_Timestamp": str(t0), "End_Timestamp": str(t0 + dt),
            "Grid_Size_X": str(grid_x)}


def test_steps_from_trace_splits_and_filters():
    """Steps are found by the embedding launch's grid (256 threads per pass
    row) and the path walk that ends a verify pass: an AR pass (1 row), a
    prefill chunk (no walk) and the weight load are left out."""
    g = "void (anonymous namespace)::gemm_kernel<unsigned short, 3, 1, 8, 2, 8, 1, true>(GemmArgs)"
    rows, t = [], 0

    def add(name, dt, grid_x=64):
        nonlocal t
        rows.append(_row(name, t, dt, grid_x))
        t += dt + 500

    for n_rows, walk in ((1, True), (17, False), (17, True), (17, True)):
        add("embed_kernel<unsigned short>(...)", 3000, 256 * n_rows)
        add(g, 30000)
        add("attn_kernel<unsigned short, 128>(AttnArgs)", 12000)
        add("attn_combine_kernel<unsigned short, 128>(...)", 5000)
        if walk:
            add("path_walk_kernel(...)", 6000)
        add("kv_compact_kernel(...)", 2000)
        add("w12_encode_kernel(...)", 9999)  # not part of a step
    steps = costmodel.steps_from_trace(rows, 17)
    assert len(steps) == 2
    for s in steps:
        assert s["gemm"] == 30.0 and s["attention"] == 17.0 and s["other"] == 11.0
        assert s.get("recurrent", 0.0) == 0.0
