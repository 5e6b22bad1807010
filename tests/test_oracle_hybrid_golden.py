"""Hand-worked pin of the oracle's recurrent (hybrid) layer wiring.

tests/golden/hybrid_mixer_case.txt works one gated diagonal recurrent layer
by hand (2 channels, 2 states, every projection a distinct small number):
the split of the input projection into [x | a | z | B | C], the state
update along each root path (a chain link and a sibling fork from the same
committed state), y = H C, the silu(z) gate and the W_out residual, through
the final norm and LM head.  The test checks the oracle against those
numbers, and checks that the plausible wiring mistakes (a and z swapped, B
and C swapped, the gate dropped, W_out transposed) each fail the comparison.
"""

import os

import numpy as np
import pytest

from oracle import Model
import oracle.model as om

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hybrid_mixer_case.txt")
F32 = np.float32


def _golden():
    vals = {"state": {}, "o": {}, "h": {}, "logits": {}}
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            f = line.split()
            if f[0] == "state":
                vals["state"][(int(f[1]), f[2])] = [float(x) for x in f[3:]]
            else:
                vals[f[0]][int(f[1])] = [float(x) for x in f[2:]]
    return vals


def _cfg():
    return dict(n_layers=1, d_model=2, n_heads=1, n_kv_heads=1, head_dim=2,
                ffn_dim=2, vocab=4, dtype="fp32", lr_state=2, layer_kinds="L",
                rms_eps=0.0, rope_theta=10000.0, name="hand_hybrid")


def _weights():
    L3 = np.log(3.0)
    w_in = np.array([[1, 0], [0, 2],          # x
                     [L3, 0], [0, L3],        # a
                     [1, 0.5], [-1, 0],       # z
                     [0.5, 0], [0, 1],        # B
                     [1, 0], [0, 3]],         # C
                    np.float64)
    return {
        "embed": np.array([[1, 1], [1, -1], [-1, 1], [2, 2]], F32),
        "layers.0.attn_norm": np.ones(2, F32),
        "layers.0.w_in": w_in.astype(F32),
        "layers.0.w_out": np.array([[1, 0], [1, 1]], F32),
        "layers.0.ffn_norm": np.ones(2, F32),
        "layers.0.wg": np.zeros((2, 2), F32),
        "layers.0.wu": np.zeros((2, 2), F32),
        "layers.0.wd": np.zeros((2, 2), F32),
        "final_norm": np.ones(2, F32),
        "lm_head": np.array([[1, 0], [0, 1], [1, 1], [1, -1]], F32),
    }


def _mismatch(model, g):
    """Largest relative deviation of the oracle from the hand-worked values
    (tree pass over nodes 0, 1, 2 plus the committed state of a chain)."""
    logits, (_, _, last_H, _) = model.forward(model.new_state(), [0, 1, 2], [-1, 0, 0],
                                              want_kv=True)
    err = 0.0
    for i in range(3):
        ref = np.array(g["logits"][i])
        err = max(err, float(np.max(np.abs(logits[i] - ref) / (np.abs(ref) + 1e-3))))
    for node in (1, 2):
        H = last_H[0][node]
        for c in (0, 1):
            ref = np.array(g["state"][(node, f"c{c}")])
            err = max(err, float(np.max(np.abs(H[c] - ref) / (np.abs(ref) + 1e-3))))
    # a chain root -> node 1 committed with append(): the committed state is
    # node 1's state
    st = model.new_state()
    model.append(st, [0, 1])
    for c in (0, 1):
        ref = np.array(g["state"][(1, f"c{c}")])
        err = max(err, float(np.max(np.abs(st.H[0][c] - ref) / (np.abs(ref) + 1e-3))))
    return err


def test_fixture_is_self_consistent():
    """The fixture's h and logits follow from its o values by the stated
    residual, W_out and final-norm arithmetic (guards the fixture itself)."""
    g = _golden()
    E = {0: [1, 1], 1: [1, -1], 2: [-1, 1]}
    for i, t in enumerate((0, 1, 2)):
        o = g["o"][i]
        h = [E[t][0] + o[0], E[t][1] + o[0] + o[1]]
        assert np.allclose(h, g["h"][i], rtol=1e-12)
        r = np.sqrt((h[0] ** 2 + h[1] ** 2) / 2)
        n = [h[0] / r, h[1] / r]
        assert np.allclose([n[0], n[1], n[0] + n[1], n[0] - n[1]], g["logits"][i],
                           rtol=1e-12)


def test_recurrent_layer_matches_hand_worked_case():
    g = _golden()
    assert _mismatch(Model(_cfg(), _weights(), max_pos=16), g) < 1e-5


def _mutant(kind):
    real = Model._recurrence

    def rec(H0, parents, x, a, z, Bm, Cm):
        if kind == "swap_a_z":
            return real(H0, parents, x, z, a, Bm, Cm)
        if kind == "swap_B_C":
            return real(H0, parents, x, a, z, Cm, Bm)
        o, H = real(H0, parents, x, a, z, Bm, Cm)
        if kind == "no_gate":
            return o / om.silu(z), H
        raise ValueError(kind)
    return staticmethod(rec)


@pytest.mark.parametrize("kind", ["swap_a_z", "swap_B_C", "no_gate", "w_out_transposed"])
def test_wiring_mistakes_fail_the_hand_worked_case(kind, monkeypatch):
    """Each plausible wiring mistake, planted in a copy of the oracle's
    recurrence on the CPU, moves the result far outside the tolerance."""
    g = _golden()
    w = _weights()
    if kind == "w_out_transposed":
        w["layers.0.w_out"] = np.ascontiguousarray(w["layers.0.w_out"].T)
    else:
        monkeypatch.setattr(Model, "_recurrence", _mutant(kind))
    assert _mismatch(Model(_cfg(), w, max_pos=16), g) > 1e-2
