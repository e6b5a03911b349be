"""The attention oracle's pins have teeth: plausible mistakes planted in a copy
of oracle/attn_oracle.py (on the CPU) are each caught by at least one pin of
tests/test_oracle_attn_pins.py."""
import types

import pytest

from oracle import attn_oracle
from tests import test_oracle_attn_pins as pins

MUTANTS = [
    ("scale dropped", "np.asarray(q_row, np.float64) * scale", "np.asarray(q_row, np.float64)"),
    ("block row t not visible to itself", "kn[b, : t + 1, g]", "kn[b, :t, g]"),
    ("block rows after t visible", "vals = np.concatenate([vc[b, :c, g], vn[b, : t + 1, g]], axis=0)",
     "vals = np.concatenate([vc[b, :c, g], vn[b, :, g]], axis=0)"),
    ("kv head by modulo", "g = h // group", "g = h % Hkv"),
    ("one context row too many", "keys = np.concatenate([kc[b, :c, g]", "keys = np.concatenate([kc[b, :c + 1, g]"),
    ("values read from the keys", "vals = np.concatenate([vc[b, :c, g], vn[b, : t + 1, g]], axis=0)",
     "vals = np.concatenate([kc[b, :c, g], kn[b, : t + 1, g]], axis=0)"),
    ("append one row late", "kc[b, c: c + T] = kn[b]", "kc[b, c + 1: c + 1 + T] = kn[b][: kc.shape[1] - c - 1]"),
    ("softmax without normalising", "return (w / w.sum()) @ np.asarray(vals, np.float64)",
     "return w @ np.asarray(vals, np.float64)"),
]

PINS = [pins.test_hand_example, pins.test_equal_scores_average_the_values, pins.test_dominant_key_selects_its_value,
        pins.test_causal_within_the_block, pins.test_context_past_ctx_is_not_read_and_order_does_not_matter,
        pins.test_grouped_query_mapping, pins.test_scale_is_applied]


def load_mutant(old, new):
    src = open(attn_oracle.__file__).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("attn_oracle_mutant")
    exec(compile(src.replace(old, new), "attn_oracle_mutant", "exec"), mod.__dict__)
    return mod


def run_pins():
    caught = []
    for pin in PINS:
        try:
            pin()
        except Exception:
            caught.append(pin.__name__)
    return caught


def test_unmutated_oracle_passes_every_pin():
    assert run_pins() == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, old, new):
    monkeypatch.setattr(pins, "A", load_mutant(old, new))
    caught = run_pins()
    print(f"{name}: caught by {caught}")
    assert caught, f"no pin catches the planted mistake: {name}"
