"""Pins of the acceptance oracle (oracle/accept_oracle.py) to facts other than
itself: hand-worked examples (tests/golden/accept_hand_examples.json) and the
defining property of exact speculative sampling -- the token it emits is
distributed exactly as the target's p, whatever the drafter's q -- checked by
integrating the oracle over grids of its uniform inputs.

Source: the audited-numbers page ("Qwen 3.8 27B mac m5: 200 tok/s, audited"),
section "How does DSpark speculative decoding create more than one token per
read?" (exact speculative sampling; greedy and sampled modes; correction and
bonus tokens; rewind of the filter history).
"""
import json
import os

import numpy as np
import pytest

from oracle import accept_oracle as A

GOLD = os.path.join(os.path.dirname(__file__), "golden", "accept_hand_examples.json")


@pytest.fixture(scope="module")
def gold():
    with open(GOLD) as f:
        return json.load(f)


def test_greedy_hand_examples(gold):
    g = gold["greedy"]
    z = np.array(g["target_logits"])[None]
    for case in g["cases"]:
        n, nxt = A.accept_greedy(z, np.array([case["drafts"]]))
        assert (int(n[0]), int(nxt[0])) == (case["n"], case["next"]), case["why"]


def test_greedy_without_drafts_emits_the_argmax():
    z = np.array([[[0.0, 1.0, 7.0, 7.0]]])
    n, nxt = A.accept_greedy(z, np.zeros((1, 0), np.int32))
    assert (int(n[0]), int(nxt[0])) == (1, 2)


def test_sampled_hand_examples(gold):
    s = gold["sampled"]
    z = np.array(s["target_logits"])[None]
    y = np.array(s["draft_logits"])[None]
    for case in s["cases"]:
        n, nxt, _ = A.accept_sampled(z, y, np.array([[case["draft"]]]), np.array([[case["u_accept"]]]),
                                     np.array([case["u_sample"]]), 1.0)
        assert (int(n[0]), int(nxt[0])) == (case["n"], case["next"]), case["why"]


def test_rewind_hand_examples(gold):
    r = gold["rewind"]
    win, rows = np.array(r["window"], np.float64), np.array(r["rows"], np.float64)
    for case in r["cases"]:
        out = A.conv_window_rewind(win, rows, np.array([case["n"]]))
        assert np.array_equal(out[0], np.array(case["out"], np.float64)), case


def test_draw_boundaries():
    w = [0.0, 0.2, 0.0, 0.5, 0.3]     # cumulative 0, .2, .2, .7, 1
    assert A.draw(w, 0.0)[0] == 1      # never a zero-weight token
    assert A.draw(w, 0.19)[0] == 1
    assert A.draw(w, 0.25)[0] == 3
    assert A.draw(w, 0.7)[0] == 4      # cumulative .7 is not above .7
    assert A.draw(w, 0.9999)[0] == 4


def _softmax(z, tau):
    e = np.exp((np.asarray(z, np.float64) - np.max(z)) / tau)
    return e / e.sum()


def _dists(seed, V):
    r = np.random.default_rng(seed)
    zt = r.normal(size=(2, V)) * 1.5   # target rows 0 and 1
    zd = r.normal(size=(1, V)) * 1.5   # drafter row 0
    return zt, zd


GRID = 2000
MID = (np.arange(GRID) + 0.5) / GRID   # midpoints: exact up to 1 / GRID per interval edge


@pytest.mark.parametrize("seed,V,tau", [(1, 4, 1.0), (2, 6, 0.7), (3, 3, 2.0)])
def test_emitted_token_is_distributed_as_the_target(seed, V, tau):
    """T = 2 (one draft).  The draft d is drawn from q; over u_accept the draft is
    kept with measure A(d); when rejected the correction is drawn over u_sample.
    P(first emitted token = x) = sum_d q(d) [A(d) 1{x = d} + (1 - A(d)) R_d(x)]
    must equal p(x); the acceptance rate sum_d q(d) A(d) must equal
    sum_x min(p(x), q(x)); a kept draft is followed by a bonus drawn from the
    next target row."""
    zt, zd = _dists(seed, V)
    p, q, p2 = _softmax(zt[0], tau), _softmax(zd[0], tau), _softmax(zt[1], tau)
    P = np.zeros(V)
    rate = 0.0
    for d in range(V):
        kept = []
        for u in MID:
            n, _, _ = A.accept_sampled(zt[None], zd[None], np.array([[d]]), np.array([[u]]), np.array([0.5]), tau)
            kept.append(n[0] == 2)
        Ad = np.mean(kept)
        rate += q[d] * Ad
        P[d] += q[d] * Ad
        if Ad < 1.0:
            u_rej = 1.0 - 0.5 / GRID        # rejected (a kept measure below 1 means p(d) < q(d))
            R = np.zeros(V)
            for u in MID:
                n, x, _ = A.accept_sampled(zt[None], zd[None], np.array([[d]]), np.array([[u_rej]]),
                                           np.array([u]), tau)
                assert n[0] == 1
                R[x[0]] += 1.0 / GRID
            P += q[d] * (1.0 - Ad) * R
        else:
            B2 = np.zeros(V)
            for u in MID:
                n, x, _ = A.accept_sampled(zt[None], zd[None], np.array([[d]]), np.array([[0.0]]),
                                           np.array([u]), tau)
                assert n[0] == 2
                B2[x[0]] += 1.0 / GRID
            assert np.abs(B2 - p2).max() <= 2.0 / GRID
    assert np.abs(P - p).max() <= 4.0 * V / GRID, (P, p)
    assert abs(rate - np.minimum(p, q).sum()) <= 2.0 / GRID


def test_sampled_with_identical_distributions_keeps_every_draft():
    """q = p makes p/q = 1: every draft is kept (u < 1) and the bonus follows."""
    r = np.random.default_rng(5)
    V, T = 7, 5
    z = r.normal(size=(1, T, V))
    d = r.integers(0, V, size=(1, T - 1))
    n, _, info = A.accept_sampled(z, z[:, : T - 1], d, np.full((1, T - 1), 0.999), np.array([0.3]), 1.0)
    assert int(n[0]) == T and info[0]["kind"] == "bonus"


def test_greedy_is_the_cold_limit_of_sampled():
    """As tau -> 0, p and q become one-hot at their argmaxes; with the drafter
    proposing its own argmax, sampled acceptance reduces to greedy."""
    r = np.random.default_rng(7)
    V, T = 9, 6
    z = r.normal(size=(3, T, V))
    y = r.normal(size=(3, T - 1, V))
    y[0] = z[0, : T - 1]                 # instance 0: drafter agrees everywhere
    d = np.argmax(y, axis=2)
    ng, xg = A.accept_greedy(z, d)
    ns, xs, _ = A.accept_sampled(z, y, d, np.full((3, T - 1), 0.5), np.full(3, 0.5), 1e-3)
    assert np.array_equal(ng, ns)
    assert int(ng[0]) == T
    # The emitted token agrees where the sampled draw is the argmax of its weights:
    # the bonus (p one-hot) always; a correction's residual max(0, p - q) is one-hot
    # at p's argmax too.
    assert np.array_equal(xg, xs)


def test_flip_matches_forcing_the_branch_through_u():
    """accept_sampled(..., flip) takes the named keep decisions the other way.  The
    same branch can be forced through the inputs: u = 0 keeps any draft with
    p(d) > 0, and u = 1e9 rejects any draft with q(d) > 0.  Both routes must give
    the same n, token and later decisions."""
    rng = np.random.default_rng(17)
    B, T, V, tau = 24, 8, 40, 1.0
    z = rng.normal(size=(B, T, V)) * 2
    y = z[:, : T - 1] + rng.normal(size=(B, T - 1, V))
    d = rng.integers(0, V, size=(B, T - 1))
    ua, us = rng.random((B, T - 1)), rng.random(B)
    _, _, info = A.accept_sampled(z, y, d, ua, us, tau)
    tried = 0
    for b in range(B):
        for j in range(len(info[b]["accept_margins"])):
            kept = j < info[b]["m"]
            u2 = ua.copy()
            u2[b, j] = 1e9 if kept else 0.0
            rn, rx, ri = A.accept_sampled(z[b:b + 1], y[b:b + 1], d[b:b + 1], u2[b:b + 1], us[b:b + 1], tau)
            fn, fx, fi = A.accept_sampled(z[b:b + 1], y[b:b + 1], d[b:b + 1], ua[b:b + 1], us[b:b + 1], tau,
                                          flip={0: {j}})
            assert (rn[0], rx[0], ri[0]["m"], ri[0]["kind"]) == (fn[0], fx[0], fi[0]["m"], fi[0]["kind"])
            if kept:
                assert fn[0] == j + 1 and fi[0]["kind"] == "correction"
            else:
                assert fn[0] >= j + 2
            tried += 1
    assert tried >= B
