"""The mixer oracle's pins have teeth: plausible mistakes planted in a copy of
oracle/mixer_oracle.py (on the CPU) are each caught by at least one pin of
tests/test_oracle_mixer_pins.py."""
import types

import pytest

from oracle import mixer_oracle
from tests import test_oracle_mixer_pins as pins

MUTANTS = [
    ("filter taps reversed", "y[:, t] += w[:, j] * full[:, t + j]", "y[:, t] += w[:, j] * full[:, t + 3 - j]"),
    ("filter without SiLU", "    y = silu(y)\n", "    y = y\n"),
    ("L2 norm over tokens", "qh = qh / np.sqrt((qh ** 2).sum(-1, keepdims=True) + EPS_L2) / np.sqrt(dk)",
     "qh = qh / np.sqrt((qh ** 2).sum(1, keepdims=True) + EPS_L2) / np.sqrt(dk)"),
    ("q not scaled", "+ EPS_L2) / np.sqrt(dk)", "+ EPS_L2)"),
    ("heads tiled instead of grouped", "q = bf16_round(np.repeat(qh, grp, axis=2))",
     "q = bf16_round(np.tile(qh, (1, 1, grp, 1)))"),
    ("decay rate without exp", "g = -np.exp(np.asarray(A_log, np.float64))", "g = -(1.0 + np.asarray(A_log, np.float64))"),
    ("softplus replaced by exp", "softplus(np.asarray(a, np.float64) + np.asarray(dt_bias, np.float64))",
     "np.exp(np.asarray(a, np.float64) + np.asarray(dt_bias, np.float64))"),
    ("beta as tanh", "beta = 1.0 / (1.0 + np.exp(-np.asarray(b, np.float64)))", "beta = np.tanh(np.asarray(b, np.float64))"),
    ("RMS over the sum", "rms = np.sqrt((o ** 2).mean(-1, keepdims=True) + EPS_RMS)",
     "rms = np.sqrt((o ** 2).sum(-1, keepdims=True) + EPS_RMS)"),
    ("output gate as sigmoid", "return o / rms * np.asarray(norm_w, np.float64) * silu(z)",
     "return o / rms * np.asarray(norm_w, np.float64) / (1.0 + np.exp(-np.asarray(z, np.float64)))"),
    ("bf16 rounding truncates", "u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000", "u = u & 0xFFFF0000"),
]

PINS = [pins.test_filter_taps_and_history_order, pins.test_unit_norms_and_q_scale,
        pins.test_value_heads_share_their_qk_head, pins.test_gate_closed_forms,
        pins.test_gated_rms_norm_closed_forms, pins.test_bf16_rounding_ties_to_even]


def load_mutant(old, new):
    src = open(mixer_oracle.__file__).read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("mixer_oracle_mutant")
    exec(compile(src.replace(old, new), "mixer_oracle_mutant", "exec"), mod.__dict__)
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
    monkeypatch.setattr(pins, "M", load_mutant(old, new))
    caught = run_pins()
    print(f"{name}: caught by {caught}")
    assert caught, f"no pin catches the planted mistake: {name}"
