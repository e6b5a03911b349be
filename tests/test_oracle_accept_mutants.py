"""The acceptance oracle's pins have teeth: plausible mistakes planted in a copy
of oracle/accept_oracle.py (on the CPU, never in the GPU path) are each caught
by at least one pin of tests/test_oracle_accept_pins.py."""
import importlib.util
import json
import os
import types

import pytest

from oracle import accept_oracle
from tests import test_oracle_accept_pins as pins

SRC = accept_oracle.__file__

# (name, original text, planted text); the original occurs exactly once.
MUTANTS = [
    ("keep test inverted to u p < q", "keep = lhs < rhs", "keep = ua[b, m] * p[tok] < q[tok]"),
    ("keep test without the drafter's q", "keep = lhs < rhs", "keep = ua[b, m] < rhs"),
    ("correction from q - p", 'w, kind = np.maximum(p - q, 0.0), "correction"',
     'w, kind = np.maximum(q - p, 0.0), "correction"'),
    ("correction drawn from p", 'w, kind = np.maximum(p - q, 0.0), "correction"', 'w, kind = p, "correction"'),
    ("bonus from the first target row", 'w, kind = softmax(z[b, T - 1], tau), "bonus"',
     'w, kind = softmax(z[b, 0], tau), "bonus"'),
    ("greedy ties take the last index", "return int(np.flatnonzero(z == z.max())[0])",
     "return int(np.flatnonzero(z == z.max())[-1])"),
    ("draw at or above instead of above", 'side="right"', 'side="left"'),
    ("n counts the kept drafts only", "        n[b] = m + 1\n        nxt[b] = x", "        n[b] = m\n        nxt[b] = x"),
    ("greedy next token from the last row", "        nxt[b] = first_argmax(z[b, m])",
     "        nxt[b] = first_argmax(z[b, T - 1])"),
    ("rewind keeps the oldest rows", "out[b] = seq[seq.shape[0] - W:]", "out[b] = seq[:W]"),
    ("temperature ignored", "x = np.asarray(z, dtype=np.float64) / float(tau)", "x = np.asarray(z, dtype=np.float64)"),
]

with open(os.path.join(os.path.dirname(__file__), "golden", "accept_hand_examples.json")) as f:
    GOLD = json.load(f)

PINS = [
    ("greedy_hand", lambda: pins.test_greedy_hand_examples(GOLD)),
    ("greedy_no_drafts", pins.test_greedy_without_drafts_emits_the_argmax),
    ("sampled_hand", lambda: pins.test_sampled_hand_examples(GOLD)),
    ("rewind_hand", lambda: pins.test_rewind_hand_examples(GOLD)),
    ("draw_boundaries", pins.test_draw_boundaries),
    ("theorem_4_1.0", lambda: pins.test_emitted_token_is_distributed_as_the_target(1, 4, 1.0)),
    ("theorem_6_0.7", lambda: pins.test_emitted_token_is_distributed_as_the_target(2, 6, 0.7)),
    ("identical_dists", pins.test_sampled_with_identical_distributions_keeps_every_draft),
    ("cold_limit", pins.test_greedy_is_the_cold_limit_of_sampled),
]


def load_mutant(old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    mod = types.ModuleType("accept_oracle_mutant")
    exec(compile(src.replace(old, new), "accept_oracle_mutant", "exec"), mod.__dict__)
    return mod


def run_pins():
    caught = []
    for name, pin in PINS:
        try:
            pin()
        except Exception:
            caught.append(name)
    return caught


def test_unmutated_oracle_passes_every_pin():
    assert run_pins() == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, old, new):
    monkeypatch.setattr(pins, "A", load_mutant(old, new))
    caught = run_pins()
    print(f"{name}: caught by {caught}")
    assert caught, f"no pin catches the planted mistake: {name}"
