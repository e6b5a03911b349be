"""The oracle's pins have teeth: plausible mistakes planted in a copy of the
oracle's C source (on the CPU, never in the GPU path) are each caught by at
least one pin of tests/test_oracle_pins.py.

Each mutant is built from the oracle's own source with one textual change, into
a temporary library that replaces the oracle's for the duration of the test.
The mistakes are the ones a reading of the recurrence
S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T, o_t = S_t q_t could
plausibly produce: a dropped decay, a wrong sign, the output read from the old
state, swapped operands, an approximated gate, and in the chunked form a
dropped decay, a wrong triangle or a missing state decay.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from oracle import gdn_oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(gdn_oracle.__file__), "gdn_oracle.c")

# (name, original text, planted text); the original occurs exactly once.
MUTANTS = [
    ("correction without the decay",
     "const double d = bt * (vt[i] - a * u);", "const double d = bt * (vt[i] - u);"),
    ("correction with the wrong sign",
     "const double d = bt * (vt[i] - a * u);", "const double d = bt * (vt[i] + a * u);"),
    ("beta on the value only",
     "const double d = bt * (vt[i] - a * u);", "const double d = bt * vt[i] - a * u;"),
    ("state not decayed",
     "Si[j] = a * Si[j] + d * kt[j];", "Si[j] = Si[j] + d * kt[j];"),
    ("output read before the rank-1 write",
     "acc += Si[j] * qt[j];", "acc += (Si[j] - d * kt[j]) * qt[j];"),
    ("output reads the key instead of the query",
     "acc += Si[j] * qt[j];", "acc += Si[j] * kt[j];"),
    ("gate linearised",
     "const double a = exp(g[row * H + h]);", "const double a = 1.0 + g[row * H + h];"),
    ("chunked: A without its decay",
     "const double A_tj = bt * exp(G[t] - G[j]) * kk;", "const double A_tj = bt * kk;"),
    ("chunked: P strictly lower instead of lower-inclusive",
     "for (int j = 0; j <= t; ++j) {\n                        const double *kj",
     "for (int j = 0; j < t; ++j) {\n                        const double *kj"),
    ("chunked: state not decayed across the chunk",
     "double s = exp(glast) * Sh[(size_t)i * dk + m];", "double s = Sh[(size_t)i * dk + m];"),
]

# Every pin, with fixed parameters where it is parametrised.
PINS = [
    ("hand_worked_example", lambda o: pins.test_hand_worked_example(o)),
    ("bruteforce_4_3_6", lambda o: pins.test_bruteforce_rational(o, 4, 3, 6)),
    ("bruteforce_2_4_3", lambda o: pins.test_bruteforce_rational(o, 2, 4, 3)),
    ("unit_decay_zero_beta", lambda o: pins.test_unit_decay_zero_beta_keeps_state(o)),
    ("delta_rule_write", lambda o: pins.test_delta_rule_writes_value(o)),
    ("zero_beta_pure_decay", lambda o: pins.test_zero_beta_is_pure_decay(o)),
    ("basis_keys", lambda o: pins.test_basis_keys_overwrite_columns(o)),
    ("chunked_C8_L37", lambda o: pins.test_chunked_equals_sequential(o, 8, 37)),
    ("chunked_C64_L130", lambda o: pins.test_chunked_equals_sequential(o, 64, 130)),
]


def build_mutant(tmp_path, old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    c = tmp_path / "mutant.c"
    c.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", *gdn_oracle.compile_flags(), str(c), "-o", str(so), "-lm"], check=True)
    return gdn_oracle.bind(ctypes.CDLL(str(so)))


def run_pins():
    caught = []
    for name, pin in PINS:
        try:
            pin(oracle)
        except Exception:  # an assertion, or the mutant rejecting its input
            caught.append(name)
    return caught


def test_unmutated_oracle_passes_every_pin(oracle_lib):
    assert run_pins() == []


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, monkeypatch, oracle_lib, name, old, new):
    monkeypatch.setattr(gdn_oracle, "_lib", build_mutant(tmp_path, old, new))
    caught = run_pins()
    print(f"{name}: caught by {caught}")
    assert caught, f"no pin catches the planted mistake: {name}"
