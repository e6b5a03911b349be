"""Pins of the GDN mixer oracle (oracle/mixer_oracle.py): closed forms of its
filter, normalisations, gates and gated RMS norm, computed here independently
(Python floats, math), chosen so that a plausible mistake (taps in the wrong
order, a missing activation, a norm over the wrong axis, the wrong head
mapping) breaks one of them.

Source: README page, "How it works" (GDN mixer row of the region table);
audited-numbers page, DSpark section (the filter's short history).  Formulas:
the published Gated DeltaNet layer (the oracle's header lists them).
"""
import math

import numpy as np
import pytest

from oracle import mixer_oracle as M

Hk, dk, H, dv = 2, 4, 4, 4
C = 2 * Hk * dk + H * dv


def silu(x):
    return x / (1.0 + math.exp(-x))


def rand(seed, B=2, T=3):
    r = np.random.default_rng(seed)
    return (r.normal(size=(B, T, C)), r.normal(size=(B, 3, C)), r.normal(size=(C, 4)), r.normal(size=(B, T, H)),
            r.normal(size=(B, T, H)), r.normal(size=H) * 0.3, r.normal(size=H) * 0.3)


def test_filter_taps_and_history_order():
    """Taps [1, 0, 0, 0] delay by three rows: output t is SiLU of history row t
    (oldest first) for t < 3, of block row t - 3 after; taps [0, 0, 0, 1] are the
    identity.  Checked on the value channels (no normalisation)."""
    x, hist, _, a, b, A_log, dtb = rand(1, B=1, T=5)
    v0 = 2 * Hk * dk
    for taps, src in (([1, 0, 0, 0], lambda t: hist[0, t] if t < 3 else x[0, t - 3]),
                      ([0, 0, 0, 1], lambda t: x[0, t])):
        w = np.tile(np.array(taps, float), (C, 1))
        _, _, v, _, _ = M.prologue(x, hist, w, a, b, A_log, dtb, Hk, dk, H, dv)
        for t in range(5):
            for c in range(H * dv):
                want = silu(float(src(t)[v0 + c]))
                got = v[0, t, c // dv, c % dv]
                assert abs(got - want) <= 2 ** -8 * abs(want) + 1e-30, (taps, t, c)


def test_unit_norms_and_q_scale():
    x, hist, w, a, b, A_log, dtb = rand(2)
    q, k, _, _, _ = M.prologue(x, hist, w, a, b, A_log, dtb, Hk, dk, H, dv)
    assert np.allclose(np.linalg.norm(k, axis=-1), 1.0, atol=2 ** -7)
    assert np.allclose(np.linalg.norm(q, axis=-1), 1.0 / math.sqrt(dk), atol=2 ** -7)


def test_value_heads_share_their_qk_head():
    """Value heads 2h and 2h + 1 read q/k head h; head 0 and head 2 differ."""
    x, hist, w, a, b, A_log, dtb = rand(3)
    q, k, _, _, _ = M.prologue(x, hist, w, a, b, A_log, dtb, Hk, dk, H, dv)
    assert np.array_equal(q[:, :, 0], q[:, :, 1]) and np.array_equal(k[:, :, 2], k[:, :, 3])
    assert not np.allclose(q[:, :, 0], q[:, :, 2])


def test_gate_closed_forms():
    x, hist, w, _, _, _, _ = rand(4, B=1, T=2)
    a = np.zeros((1, 2, H))
    b = np.zeros((1, 2, H))
    a[0, 1] = -60.0                          # softplus(-60) ~ 0: no decay
    _, _, _, g, beta = M.prologue(x, hist, w, a, b, np.zeros(H), np.zeros(H), Hk, dk, H, dv)
    assert np.allclose(g[0, 0], -math.log(2.0), atol=1e-15)
    assert np.all(np.abs(g[0, 1]) < 1e-25)
    assert np.allclose(beta, 0.5)
    _, _, _, g2, _ = M.prologue(x, hist, w, a, b, np.full(H, math.log(3.0)), np.zeros(H), Hk, dk, H, dv)
    assert np.allclose(g2[0, 0], -3.0 * math.log(2.0), atol=1e-14)


def test_gated_rms_norm_closed_forms():
    r = np.random.default_rng(5)
    z = r.normal(size=(1, 1, 2, dv))
    nw = r.normal(size=dv)
    o = np.zeros((1, 1, 2, dv))
    o[0, 0, 0] = 3.0                        # a constant row c: normalised to c / sqrt(c^2 + eps)
    o[0, 0, 1] = -0.25
    y = M.epilogue(o, z, nw)
    for hh, c in ((0, 3.0), (1, -0.25)):
        want = [c / math.sqrt(c * c + 1e-6) * nw[i] * silu(z[0, 0, hh, i]) for i in range(dv)]
        assert np.allclose(y[0, 0, hh], want, rtol=1e-12)
    o2 = r.normal(size=(1, 1, 2, dv))
    assert np.allclose(M.epilogue(o2 * 7.0, z, nw), M.epilogue(o2, z, nw), rtol=1e-6)


def test_bf16_rounding_ties_to_even():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20])
    want = np.array([1.0, 1.0, 1 + 2 ** -6, -1.0, 1 + 2 ** -7])
    assert np.array_equal(M.bf16_round(vals), want)
