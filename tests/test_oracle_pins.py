"""Pins of the fp64 oracle against what the recurrence's definition fixes.

The recurrence is the gated delta rule of the GDN mixer (lithos-metal README,
"How it works", region table, "GDN mixer" row; update rule from Gated
DeltaNet, ICLR 2025):  S_t = a_t S_{t-1}(I - b_t k_t k_t^T) + b_t v_t k_t^T,
o_t = S_t q_t.  None of these tests re-types the oracle's loop: each checks a
closed form, an exact rational evaluation in another association, a
hand-worked example, or an invariant.  dk != dv wherever the case allows, so a
transposed state would fail.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from tests import _bruteforce as bf

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, B=2, H=3, dk=8, dv=5, L=12, unit_k=True):
    S0 = rng.normal(size=(B, H, dv, dk)) * 0.3
    q = rng.normal(size=(B, L, H, dk))
    k = rng.normal(size=(B, L, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.normal(size=(B, L, H, dv))
    g = -np.log1p(np.exp(rng.normal(size=(B, L, H))))
    beta = 1.0 / (1.0 + np.exp(-rng.normal(size=(B, L, H))))
    return S0, q, k, v, g, beta


def states_all(oracle_lib, S0, q, k, v, g, beta):
    """S_0..S_L via the commit entry (keep = n for every n)."""
    B, L = q.shape[0], q.shape[1]
    return [oracle_lib.commit(S0, q, k, v, g, beta, np.full(B, n, np.int32)) for n in range(L + 1)]


# --- hand-worked example -------------------------------------------------------

def test_hand_worked_example(oracle_lib):
    """Values worked by hand (tests/golden/hand_example_dk2_dv3.json)."""
    ex = json.load(open(os.path.join(GOLDEN, "hand_example_dk2_dv3.json")))
    F = lambda m: np.array([[float(Fraction(x)) for x in r] for r in m])
    S0 = F(ex["S0"])[None, None]
    a = np.array([float(Fraction(x)) for x in ex["a"]])
    T = len(a)
    g = np.log(a).reshape(1, T, 1)
    beta = np.array([float(Fraction(x)) for x in ex["beta"]]).reshape(1, T, 1)
    k = F(ex["k"]).reshape(1, T, 1, 2)
    q = F(ex["q"]).reshape(1, T, 1, 2)
    v = F(ex["v"]).reshape(1, T, 1, 3)
    o, S2 = oracle_lib.prefill_seq(S0, q, k, v, g, beta)
    S1 = oracle_lib.commit(S0, q, k, v, g, beta, np.array([1], np.int32))
    np.testing.assert_allclose(o[0, :, 0], F(ex["expected_o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(S1[0, 0], F(ex["expected_S1"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(S2[0, 0], F(ex["expected_S2"]), rtol=0, atol=1e-14)
    # The same example through the exact rational recurrence.
    Fr = lambda m: [[Fraction(x) for x in r] for r in m]
    states, outs = bf.recurrence(Fr(ex["S0"]), [Fraction(x) for x in ex["a"]],
                                 [Fraction(x) for x in ex["beta"]], Fr(ex["k"]), Fr(ex["v"]),
                                 Fr(ex["q"]))
    assert states[0] == Fr(ex["expected_S1"]) and states[1] == Fr(ex["expected_S2"])
    assert outs == Fr(ex["expected_o"])


# --- exact rational brute force -------------------------------------------------

@pytest.mark.parametrize("dk,dv,T", [(4, 4, 5), (4, 3, 6), (2, 4, 3)])
def test_bruteforce_rational(oracle_lib, dk, dv, T):
    """1 head, tiny dims, rational inputs: exact recurrence in the literal matrix
    form vs the oracle's row-wise fp64 loop."""
    rng = np.random.default_rng(100 + dk * 10 + dv)
    rint = lambda lo, hi: Fraction(int(rng.integers(lo, hi)), 8)
    S0 = [[rint(-16, 17) for _ in range(dk)] for _ in range(dv)]
    k = [[rint(-8, 9) for _ in range(dk)] for _ in range(T)]
    q = [[rint(-8, 9) for _ in range(dk)] for _ in range(T)]
    v = [[rint(-16, 17) for _ in range(dv)] for _ in range(T)]
    a = [Fraction(int(rng.integers(1, 9)), 8) for _ in range(T)]
    beta = [Fraction(int(rng.integers(0, 9)), 8) for _ in range(T)]
    states, outs = bf.recurrence(S0, a, beta, k, v, q)
    f = lambda m: np.array(m, dtype=np.float64)
    o, S = oracle_lib.prefill_seq(f(S0)[None, None], f(q).reshape(1, T, 1, dk),
                                  f(k).reshape(1, T, 1, dk), f(v).reshape(1, T, 1, dv),
                                  np.log(f(a)).reshape(1, T, 1), f(beta).reshape(1, T, 1))
    ref_o = np.array([[float(x) for x in r] for r in outs])
    ref_S = np.array([[float(x) for x in r] for r in states[-1]])
    scale = max(1.0, np.abs(ref_o).max())
    np.testing.assert_allclose(o[0, :, 0], ref_o, rtol=0, atol=1e-13 * scale)
    np.testing.assert_allclose(S[0, 0], ref_S, rtol=0, atol=1e-13 * max(1.0, np.abs(ref_S).max()))
    for n in range(T + 1):
        Sn = oracle_lib.commit(f(S0)[None, None], f(q).reshape(1, T, 1, dk),
                               f(k).reshape(1, T, 1, dk), f(v).reshape(1, T, 1, dv),
                               np.log(f(a)).reshape(1, T, 1), f(beta).reshape(1, T, 1),
                               np.array([n], np.int32))
        ref = f(S0) if n == 0 else np.array([[float(x) for x in r] for r in states[n - 1]])
        np.testing.assert_allclose(Sn[0, 0], ref, rtol=0, atol=1e-13 * max(1.0, np.abs(ref).max()))


# --- closed forms ---------------------------------------------------------------

def test_unit_decay_zero_beta_keeps_state(oracle_lib):
    """g = 0 (a = 1) and beta = 0: S_t == S0 bit for bit and o_t = S0 q_t."""
    rng = np.random.default_rng(1)
    S0, q, k, v, g, beta = rand_case(rng)
    g[:] = 0.0
    beta[:] = 0.0
    o, S = oracle_lib.prefill_seq(S0, q, k, v, g, beta)
    assert np.array_equal(S, S0)
    ref = np.einsum("bhij,blhj->blhi", S0, q)
    np.testing.assert_allclose(o, ref, rtol=0, atol=1e-14)


def test_delta_rule_writes_value(oracle_lib):
    """a = 1, beta = 1, |k| = 1: the updated state maps k_t exactly to v_t, so
    S_t k_t = v_t; with q_t = k_t the output is v_t."""
    rng = np.random.default_rng(2)
    S0, q, k, v, g, beta = rand_case(rng, L=9)
    g[:] = 0.0
    beta[:] = 1.0
    states = states_all(oracle_lib, S0, q, k, v, g, beta)
    for t in range(q.shape[1]):
        St = states[t + 1]
        np.testing.assert_allclose(np.einsum("bhij,bhj->bhi", St, k[:, t]), v[:, t],
                                   rtol=0, atol=1e-13)
    o, _ = oracle_lib.prefill_seq(S0, k, k, v, g, beta)
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-13)


def test_zero_beta_is_pure_decay(oracle_lib):
    """beta = 0: S_t = exp(G_t) S0 with G_t the running sum of g, and
    o_t = exp(G_t) S0 q_t."""
    rng = np.random.default_rng(3)
    S0, q, k, v, g, beta = rand_case(rng)
    beta[:] = 0.0
    G = np.cumsum(g, axis=1)                        # [B][L][H]
    states = states_all(oracle_lib, S0, q, k, v, g, beta)
    for t in range(q.shape[1]):
        ref = np.exp(G[:, t])[:, :, None, None] * S0
        np.testing.assert_allclose(states[t + 1], ref, rtol=1e-13, atol=1e-15)
    o, _ = oracle_lib.prefill_seq(S0, q, k, v, g, beta)
    ref_o = np.exp(G)[..., None] * np.einsum("bhij,blhj->blhi", S0, q)
    np.testing.assert_allclose(o, ref_o, rtol=1e-13, atol=1e-15)


def test_basis_keys_overwrite_columns(oracle_lib):
    """a = 1, beta = 1, k_t = e_t: each step replaces column t of S by v_t, so
    S_T is S0 with columns 0..T-1 replaced by v_0..v_{T-1}."""
    rng = np.random.default_rng(4)
    B, H, dk, dv, T = 2, 2, 8, 5, 6
    S0, q, _, v, g, beta = rand_case(rng, B, H, dk, dv, T)
    k = np.zeros((B, T, H, dk))
    for t in range(T):
        k[:, t, :, t] = 1.0
    g[:] = 0.0
    beta[:] = 1.0
    _, S = oracle_lib.prefill_seq(S0, q, k, v, g, beta)
    ref = S0.copy()
    for t in range(T):
        ref[:, :, :, t] = v[:, t]
    np.testing.assert_allclose(S, ref, rtol=0, atol=1e-15)


# --- invariants -----------------------------------------------------------------

def test_joint_linearity_in_state_and_values(oracle_lib):
    """(S0, v) -> (S_t, o_t) is linear for fixed q, k, g, beta."""
    rng = np.random.default_rng(5)
    S1, q, k, v1, g, beta = rand_case(rng)
    S2 = rng.normal(size=S1.shape)
    v2 = rng.normal(size=v1.shape)
    alpha = -1.75
    o1, F1 = oracle_lib.prefill_seq(S1, q, k, v1, g, beta)
    o2, F2 = oracle_lib.prefill_seq(S2, q, k, v2, g, beta)
    o3, F3 = oracle_lib.prefill_seq(alpha * S1 + S2, q, k, alpha * v1 + v2, g, beta)
    np.testing.assert_allclose(o3, alpha * o1 + o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(F3, alpha * F1 + F2, rtol=0, atol=1e-12)


def test_value_row_permutation(oracle_lib):
    """Permuting value rows of (S0, v) permutes the rows of S and o: rows never mix,
    which is what lets the state be split by value index."""
    rng = np.random.default_rng(6)
    S0, q, k, v, g, beta = rand_case(rng)
    perm = rng.permutation(S0.shape[2])
    o, S = oracle_lib.prefill_seq(S0, q, k, v, g, beta)
    op, Sp = oracle_lib.prefill_seq(S0[:, :, perm], q, k, v[..., perm], g, beta)
    assert np.array_equal(op, o[..., perm])
    assert np.array_equal(Sp, S[:, :, perm])


def test_transition_is_non_expansive(oracle_lib):
    """For a in (0,1], beta in [0,2], |k| <= 1, S -> a S (I - beta k k^T) has norm
    <= 1, so two runs from different states on the same inputs never move apart.
    A sign error in the beta term (I + beta k k^T) would break this."""
    rng = np.random.default_rng(7)
    S0, q, k, v, g, beta = rand_case(rng, B=1, H=2, dk=6, dv=4, L=60)
    beta = 2.0 * beta
    g = 0.02 * g  # slow decay, so the distance stays far above rounding
    S0b = S0 + rng.normal(size=S0.shape)
    sa = states_all(oracle_lib, S0, q, k, v, g, beta)
    sb = states_all(oracle_lib, S0b, q, k, v, g, beta)
    # Frobenius distance per head: |D M|_F <= |D|_F |M|_2 <= |D|_F.
    dist = np.array([np.linalg.norm(x - y, axis=(2, 3)) for x, y in zip(sa, sb)])
    assert dist[-1].min() > 1e-3
    for t in range(1, len(dist)):
        assert np.all(dist[t] <= dist[t - 1] * (1 + 1e-12))
    # The same check with the sign of the beta term flipped must fail, so the
    # test can see such a mistake: |I + beta k k^T| > 1.
    kk = k[0, 0, 0]
    M_bad = np.eye(6) + beta[0, 0, 0] * np.outer(kk, kk)
    assert np.linalg.norm(M_bad, 2) > 1.0


def test_causality(oracle_lib):
    """Outputs o_1..o_t do not depend on rows after t (bit for bit)."""
    rng = np.random.default_rng(8)
    S0, q, k, v, g, beta = rand_case(rng, L=10)
    o, _ = oracle_lib.prefill_seq(S0, q, k, v, g, beta)
    t = 4
    q2, k2, v2, g2, b2 = (x.copy() for x in (q, k, v, g, beta))
    for x in (q2, k2, v2):
        x[:, t + 1:] = rng.normal(size=x[:, t + 1:].shape)
    g2[:, t + 1:] -= 0.5
    b2[:, t + 1:] = 0.3
    o2, _ = oracle_lib.prefill_seq(S0, q2, k2, v2, g2, b2)
    assert np.array_equal(o2[:, : t + 1], o[:, : t + 1])


# --- commit and chunked form ----------------------------------------------------

def test_commit_zero_is_identity_bytes(oracle_lib):
    rng = np.random.default_rng(9)
    S0, q, k, v, g, beta = rand_case(rng)
    S0[0, 0, 0, 0] = -0.0
    S = oracle_lib.commit(S0, q, k, v, g, beta, np.zeros(S0.shape[0], np.int32))
    assert S.tobytes() == np.ascontiguousarray(S0).tobytes()


def test_commit_n_equals_prefill_of_n_tokens(oracle_lib):
    """commit(n) of a block = prefill of its first n rows; verify + commit(T) =
    prefill of the whole block (outputs and state)."""
    rng = np.random.default_rng(10)
    S0, q, k, v, g, beta = rand_case(rng, B=3, L=8)
    n = np.array([3, 8, 5], np.int32)
    S = oracle_lib.commit(S0, q, k, v, g, beta, n)
    for b in range(3):
        sl = lambda x: x[b:b + 1, : n[b]]
        _, Sp = oracle_lib.prefill_seq(S0[b:b + 1], sl(q), sl(k), sl(v), sl(g), sl(beta))
        assert np.array_equal(S[b:b + 1], Sp)
    o = oracle_lib.verify(S0, q, k, v, g, beta)
    op, Sp = oracle_lib.prefill_seq(S0, q, k, v, g, beta)
    ST = oracle_lib.commit(S0, q, k, v, g, beta, np.full(3, 8, np.int32))
    assert np.array_equal(o, op) and np.array_equal(ST, Sp)


def test_prompt_split_is_exact(oracle_lib):
    """prefill(L1) then prefill(L2) == prefill(L1 + L2)."""
    rng = np.random.default_rng(11)
    S0, q, k, v, g, beta = rand_case(rng, L=20)
    o, S = oracle_lib.prefill_seq(S0, q, k, v, g, beta)
    cut = 7
    a = lambda x: x[:, :cut]
    z = lambda x: x[:, cut:]
    o1, S1 = oracle_lib.prefill_seq(S0, a(q), a(k), a(v), a(g), a(beta))
    o2, S2 = oracle_lib.prefill_seq(S1, z(q), z(k), z(v), z(g), z(beta))
    assert np.array_equal(np.concatenate([o1, o2], axis=1), o) and np.array_equal(S2, S)


@pytest.mark.parametrize("C", [1, 2, 3, 8, 64])
@pytest.mark.parametrize("L", [37, 130])
def test_chunked_equals_sequential(oracle_lib, C, L):
    """The UT/WY chunk form reaches the sequential result (tail chunks included)."""
    rng = np.random.default_rng(12 + C + L)
    S0, q, k, v, g, beta = rand_case(rng, B=1, H=2, dk=8, dv=6, L=L)
    o, S = oracle_lib.prefill_seq(S0, q, k, v, g, beta)
    oc, Sc = oracle_lib.prefill_chunked(S0, q, k, v, g, beta, C)
    np.testing.assert_allclose(oc, o, rtol=0, atol=1e-12 * np.abs(o).max())
    np.testing.assert_allclose(Sc, S, rtol=0, atol=1e-12 * np.abs(S).max())


def test_chunk_of_one_reduces_to_step(oracle_lib):
    """With C = 1 the chunk form is the single step: Tm = beta, W = beta a k,
    D = beta (v - a S k), O = a S q + (q.k) D, S <- a S + D k^T."""
    rng = np.random.default_rng(13)
    S0, q, k, v, g, beta = rand_case(rng, B=1, H=1, dk=5, dv=3, L=1)
    a = np.exp(g[0, 0, 0])
    bt = beta[0, 0, 0]
    s, kk, qq, vv = S0[0, 0], k[0, 0, 0], q[0, 0, 0], v[0, 0, 0]
    D = bt * (vv - a * s @ kk)
    ref_o = a * s @ qq + (qq @ kk) * D
    ref_S = a * s + np.outer(D, kk)
    oc, Sc = oracle_lib.prefill_chunked(S0, q, k, v, g, beta, 1)
    np.testing.assert_allclose(oc[0, 0, 0], ref_o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(Sc[0, 0], ref_S, rtol=0, atol=1e-14)


def test_bad_arguments_rejected(oracle_lib):
    rng = np.random.default_rng(14)
    S0, q, k, v, g, beta = rand_case(rng, B=2, L=4)
    with pytest.raises(ValueError):
        oracle_lib.commit(S0, q, k, v, g, beta, np.array([5, 0], np.int32))
