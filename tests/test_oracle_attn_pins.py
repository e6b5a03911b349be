"""Pins of the full-attention oracle (oracle/attn_oracle.py): a hand-worked
example (tests/golden/attn_hand_example.json) and closed forms and invariants of
softmax attention that a plausible mistake (a missing scale, a wrong causal
bound, a wrong grouped-query mapping, rows past the context read) breaks.

Source: README page, "How it works" (full-attention mixer); audited-numbers page,
"How does lithos-metal fuse layer mixers on Metal?".
"""
import json
import os

import numpy as np
import pytest

from oracle import attn_oracle as A

GOLD = os.path.join(os.path.dirname(__file__), "golden", "attn_hand_example.json")


def rand_case(seed, B=2, T=4, Hq=4, Hkv=2, d=8, Lmax=12, ctx=(5, 0)):
    r = np.random.default_rng(seed)
    q = r.normal(size=(B, T, Hq, d))
    kn, vn = r.normal(size=(B, T, Hkv, d)), r.normal(size=(B, T, Hkv, d))
    kc, vc = r.normal(size=(B, Lmax, Hkv, d)), r.normal(size=(B, Lmax, Hkv, d))
    return q, kn, vn, kc, vc, np.array(ctx)


def test_hand_example():
    g = json.load(open(GOLD))
    o, kc, vc = A.attn_verify(g["q"], g["k_new"], g["v_new"], g["k_cache"], g["v_cache"], g["ctx"], g["scale"])
    assert np.abs(o - np.array(g["o"])).max() < 1e-12
    # The block's rows are appended at ctx .. ctx+T-1.
    assert np.array_equal(kc[0, 2:4], np.array(g["k_new"])[0])
    assert np.array_equal(vc[0, 2:4], np.array(g["v_new"])[0])


def test_equal_scores_average_the_values():
    """Identical keys give equal weights: each output is the mean of the values
    it may see (the context and block rows 0 .. t)."""
    q, kn, vn, kc, vc, ctx = rand_case(1)
    kn[:] = 0.7
    kc[:] = 0.7
    o, _, _ = A.attn_verify(q, kn, vn, kc, vc, ctx, 0.3)
    B, T, Hq, d = q.shape
    for b in range(B):
        for t in range(T):
            for h in range(Hq):
                g = h // (Hq // kn.shape[2])
                vals = np.concatenate([vc[b, : ctx[b], g], vn[b, : t + 1, g]])
                assert np.allclose(o[b, t, h], vals.mean(axis=0), atol=1e-12)


def test_dominant_key_selects_its_value():
    """One key aligned with the query at a huge scale takes all the weight."""
    q, kn, vn, kc, vc, ctx = rand_case(2, B=1, ctx=(6,))
    d = q.shape[-1]
    q[:] = 0.0
    q[..., 0] = 1.0
    kc[:] = 0.0
    kn[:] = 0.0
    kc[0, 3, :, 0] = 1.0          # context row 3, every kv head
    o, _, _ = A.attn_verify(q, kn, vn, kc, vc, ctx, 200.0)
    for h in range(q.shape[2]):
        g = h // (q.shape[2] // kn.shape[2])
        assert np.allclose(o[0, :, h], vc[0, 3, g], atol=1e-12)


def test_causal_within_the_block():
    """Row t's output does not depend on block rows after t."""
    q, kn, vn, kc, vc, ctx = rand_case(3)
    o1, _, _ = A.attn_verify(q, kn, vn, kc, vc, ctx, 0.4)
    kn2, vn2 = kn.copy(), vn.copy()
    kn2[:, 2:] += 5.0
    vn2[:, 2:] -= 3.0
    o2, _, _ = A.attn_verify(q, kn2, vn2, kc, vc, ctx, 0.4)
    assert np.array_equal(o1[:, :2], o2[:, :2])
    assert not np.allclose(o1[:, 2:], o2[:, 2:])


def test_context_past_ctx_is_not_read_and_order_does_not_matter():
    q, kn, vn, kc, vc, ctx = rand_case(4)
    o1, _, _ = A.attn_verify(q, kn, vn, kc, vc, ctx, 0.5)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[0, ctx[0]:] = 1e3                      # junk past the context
    perm = np.random.default_rng(9).permutation(ctx[0])
    kc2[0, : ctx[0]] = kc[0, perm]
    vc2[0, : ctx[0]] = vc[0, perm]
    o2, _, _ = A.attn_verify(q, kn, vn, kc2, vc2, ctx, 0.5)
    assert np.allclose(o1, o2, atol=1e-12)


def test_grouped_query_mapping():
    """Query heads of one group share a key/value head: swapping the two kv heads
    equals swapping the two groups of query heads."""
    q, kn, vn, kc, vc, ctx = rand_case(5, Hq=4, Hkv=2)
    o1, _, _ = A.attn_verify(q, kn, vn, kc, vc, ctx, 0.5)
    sw = lambda x: x[:, :, ::-1].copy()
    qs = q[:, :, [2, 3, 0, 1]].copy()
    o2, _, _ = A.attn_verify(qs, sw(kn), sw(vn), sw(kc), sw(vc), ctx, 0.5)
    assert np.allclose(o1, o2[:, :, [2, 3, 0, 1]], atol=1e-12)


def test_scale_is_applied():
    """Scale 0 averages uniformly; a nonzero scale does not."""
    q, kn, vn, kc, vc, ctx = rand_case(6)
    o0, _, _ = A.attn_verify(q, kn, vn, kc, vc, ctx, 0.0)
    ob, _, _ = A.attn_verify(q, kn, vn, kc, vc, ctx, 1.0)
    b, t, h = 0, 1, 0
    vals = np.concatenate([vc[b, : ctx[b], 0], vn[b, : t + 1, 0]])
    assert np.allclose(o0[b, t, h], vals.mean(axis=0), atol=1e-12)
    assert not np.allclose(ob[b, t, h], vals.mean(axis=0))
