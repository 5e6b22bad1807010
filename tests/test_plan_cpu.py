"""Batched draft planner (host code of the C-ABI library): the length rule,
the shared budget, optimality against brute force, and the acceptance
estimate (CPU only)."""

import itertools
import math

import numpy as np
import pytest

from tree_verification_spec_amd import (SpecError, SPEC_E_INVAL, spec_acceptance_update,
                                        spec_plan_drafts)


def _rate(s, f):
    return (s + 1.0) / (s + f + 2.0)


def _length_rule(p, choices, min_prob):
    ok = [c for c in choices if p ** c >= min_prob]
    return max(ok) if ok else min(choices)


def _gain(ps, lens):
    return sum(sum(p ** j for j in range(1, L + 1)) for p, L in zip(ps, lens))


def test_length_rule_without_budget_pressure():
    succ = [0.0, 3.0, 20.0, 200.0]
    fail = [9.0, 3.0, 2.0, 1.0]
    lens = spec_plan_drafts(succ, fail, [8, 12, 16], 0.05, 10_000)
    ps = [_rate(s, f) for s, f in zip(succ, fail)]
    assert lens == [_length_rule(p, [8, 12, 16], 0.05) for p in ps]
    assert lens[-1] == 16 and lens[0] == 8


def test_budget_prefixes_and_optimality_against_brute_force():
    rng = np.random.default_rng(5)
    choices = [1, 2, 4]
    for trial in range(60):
        n = int(rng.integers(1, 5))
        succ = list(rng.uniform(0, 30, n).round(2))
        fail = list(rng.uniform(0, 10, n).round(2))
        budget = int(rng.integers(0, 12))
        lens = spec_plan_drafts(succ, fail, choices, 0.05, budget)
        ps = [_rate(s, f) for s, f in zip(succ, fail)]
        caps = [_length_rule(p, choices, 0.05) for p in ps]
        assert sum(lens) <= budget
        assert all(0 <= L <= c for L, c in zip(lens, caps))
        assert sum(lens) == min(budget, sum(caps))
        # the kept positions maximise the expected accepted positions
        best = max(_gain(ps, ls) for ls in itertools.product(*[range(c + 1) for c in caps])
                   if sum(ls) <= budget)
        assert _gain(ps, lens) == pytest.approx(best, rel=1e-9, abs=1e-12)


def test_budget_ties_go_to_lower_requests_then_positions():
    # equal estimates: positions are handed out round by round
    lens = spec_plan_drafts([4.0] * 3, [4.0] * 3, [4], 0.0, 7)
    assert lens == [3, 2, 2]
    assert spec_plan_drafts([4.0] * 3, [4.0] * 3, [4], 0.0, 0) == [0, 0, 0]


def test_acceptance_update_and_estimate():
    s, f = spec_acceptance_update([8, 8, 0], [8, 3, 0], 0.5, [2.0, 2.0, 2.0], [4.0, 4.0, 4.0])
    assert s == [9.0, 4.0, 1.0] and f == [2.0, 3.0, 2.0]  # offering nothing fails nothing
    # chains whose positions match independently with probability a: the
    # undecayed estimate converges to a (successes over successes + failures
    # is the estimate of a geometric run's continuation probability)
    rng = np.random.default_rng(11)
    for a in (0.3, 0.7, 0.9):
        succ, fail = [0.0], [0.0]
        for _ in range(4000):
            hits = rng.random(8) < a
            acc = 8 if hits.all() else int(np.argmin(hits))
            succ, fail = spec_acceptance_update([8], [acc], 1.0, succ, fail)
        assert _rate(succ[0], fail[0]) == pytest.approx(a, abs=0.02)


def test_invalid_arguments():
    with pytest.raises(SpecError) as e:
        spec_acceptance_update([3], [4], 0.9, [0.0], [0.0])
    assert e.value.code == SPEC_E_INVAL
    with pytest.raises(SpecError):
        spec_acceptance_update([3], [1], 1.5, [0.0], [0.0])
    with pytest.raises(SpecError):
        spec_plan_drafts([1.0], [1.0], [0], 0.05, 4)
    with pytest.raises(SpecError):
        spec_plan_drafts([1.0], [1.0], [8], 0.05, -1)
    with pytest.raises(SpecError):
        spec_plan_drafts([-1.0], [1.0], [8], 0.05, 4)
    assert spec_plan_drafts([], [], [8], 0.05, 4) == []
