"""Pins of the generation-loop contract (oracle/generate.py).

The loop runs on a scripted stand-in model whose every prediction is fixed,
so each expectation below is worked out by hand from the contract ("Coming
back to Failed Star", section "Next: one complete deterministic generation
arc"): zero budget, EOS on the first step (with and without the stop ID),
the budget, both sides of the context boundary, an exact logit tie.
"""
import numpy as np
import pytest

from oracle import generate as G

V = 16


class Script:
    """Predicts next[pos] from position pos; records every forward."""

    def __init__(self, nxt, tie=None):
        self.nxt = dict(nxt)
        self.calls = []
        self.tie = tie or {}

    def _logits(self, pos):
        lg = np.full(V, -1.0)
        lg[self.nxt.get(pos, 0)] = 1.0
        for t in self.tie.get(pos, ()):
            lg[t] = 1.0
        return lg

    def prefill(self, prompt):
        self.calls.append(("prefill", len(prompt)))
        return self._logits(len(prompt) - 1)

    def decode(self, tok, pos):
        self.calls.append(("decode", tok, pos))
        return self._logits(pos)


def run(sc, prompt, budget, max_ctx, eos=(), inc=False):
    return G.generate_loop(sc.prefill, sc.decode, prompt, budget, max_ctx, eos, inc)


def test_zero_budget_runs_nothing():
    sc = Script({})
    assert run(sc, [1, 2, 3], 0, 32) == ([], G.STOP_BUDGET)
    assert sc.calls == []


def test_empty_and_oversized_prompt_are_errors():
    with pytest.raises(ValueError):
        run(Script({}), [], 4, 32)
    with pytest.raises(ValueError):
        run(Script({}), list(range(33)), 4, 32)


def test_eos_on_first_step():
    sc = Script({2: 7})
    assert run(sc, [1, 2, 3], 5, 32, eos=(7, 9)) == ([], G.STOP_EOS)
    assert sc.calls == [("prefill", 3)]
    assert run(Script({2: 7}), [1, 2, 3], 5, 32, eos=(7,), inc=True) == ([7], G.STOP_EOS)


def test_budget_stops_without_an_extra_forward():
    sc = Script({2: 4, 3: 5, 4: 6, 5: 8})
    assert run(sc, [1, 2, 3], 3, 32) == ([4, 5, 6], G.STOP_BUDGET)
    assert sc.calls == [("prefill", 3), ("decode", 4, 3), ("decode", 5, 4)]


def test_eos_after_some_tokens():
    sc = Script({2: 4, 3: 5, 4: 9})
    assert run(sc, [1, 2, 3], 10, 32, eos=(9,)) == ([4, 5], G.STOP_EOS)


def test_context_boundary_both_sides():
    # S = 3, max_ctx = 5: forwards at positions 3 and 4 are allowed, 5 is not
    sc = Script({2: 4, 3: 5, 4: 6, 5: 7})
    assert run(sc, [1, 2, 3], 10, 5) == ([4, 5, 6], G.STOP_CONTEXT)
    assert [c[2] for c in sc.calls if c[0] == "decode"] == [3, 4]
    # the same run with a budget of exactly three tokens ends on the budget
    assert run(Script({2: 4, 3: 5, 4: 6}), [1, 2, 3], 3, 5) == ([4, 5, 6], G.STOP_BUDGET)
    # a prompt that fills the context returns the one token its logits predict
    sc = Script({4: 11})
    assert run(sc, [1, 2, 3, 4, 5], 10, 5) == ([11], G.STOP_CONTEXT)
    assert sc.calls == [("prefill", 5)]


def test_exact_tie_selects_lowest_id():
    sc = Script({2: 9}, tie={2: (4,)})
    assert run(sc, [1, 2, 3], 1, 32) == ([4], G.STOP_BUDGET)
