"""GPU parity of gdn_verify_block and gdn_commit against the fp64 oracle.

Every call goes through libgdn's C ABI (via the ctypes binding).  Bars:
outputs within 2e-3 and committed states within 1e-3 (worst (instance, head)
slab, max|x - r| / max|r|), the accepted-prefix selection exact (pos advances
by exactly n, the state matches S_n and not its neighbours), commit(0)
byte-identical, causality and run-to-run determinism bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from speculative_verify_amd.inputs import make_accepts, make_inputs
from tests._metrics import OUT_TOL, STATE_TOL, rel_err_outputs, rel_err_state

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def G():
    import speculative_verify_amd.gdn as G
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    return G


def run_verify(G, x, record=None):
    B, H, dk, dv, T = x.shape
    o = torch.empty(B, T, H, dv, dtype=torch.float32, device=DEV)
    if record is None:
        record = G.new_record(x.S0, T, x.q.dtype)
    G.gdn_verify_block(x.S0, x.q, x.k, x.v, x.g, x.beta, o, record)
    return o, record


def oracle_states(x, T):
    """S_0..S_T from the oracle (float64 numpy)."""
    B = x.S0.shape[0]
    xc = x.to("cpu")
    return [oracle.commit(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta, np.full(B, n, np.int32))
            for n in range(T + 1)]


def print_case(**kw):
    print("case:", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


# --- the tiny fp32 verify: 1 layer, 2 heads, d = 64, T = 8 ------------------------

def test_tiny_fp32_block_all_n(G):
    print_case(test="tiny_fp32", B=1, H=2, d=64, T=8, seed=0)
    x = make_inputs(1, 2, 64, 64, 8, dtype=torch.float32, seed=0, device=DEV)
    xc = x.to("cpu")
    o, rec = run_verify(G, x)
    ref_o = oracle.verify(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta)
    assert rel_err_outputs(o, ref_o) <= OUT_TOL
    states = oracle_states(x, 8)
    S_ckpt = x.S0.clone()
    for n in range(9):
        S = S_ckpt.clone()
        o, rec = run_verify(G, x.__class__(S, x.q, x.k, x.v, x.g, x.beta), rec)
        pos = torch.tensor([100], dtype=torch.int32, device=DEV)
        G.gdn_commit(S, rec, torch.tensor([n], dtype=torch.int32, device=DEV), pos)
        torch.cuda.synchronize()
        assert int(pos.item()) == 100 + n
        if n == 0:
            assert torch.equal(S.view(torch.int32), S_ckpt.view(torch.int32))
        err = rel_err_state(S, states[n])
        assert err <= STATE_TOL, (n, err)
        # The selection is exact: S is far closer to S_n than to its neighbours.
        for m in (n - 1, n + 1):
            if 0 <= m <= 8:
                gap = rel_err_state(states[m], states[n])
                if gap > 10 * STATE_TOL:
                    assert rel_err_state(S, states[m]) > 10 * err
        assert G.gdn_record_status(rec, S) == [0]


# --- bf16 blocks over the supported shapes and block lengths -----------------------

@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [1, 3, 8, 16])
def test_bf16_shapes(G, dk, dv, T):
    B, H = 3, 5
    print_case(test="bf16_shapes", B=B, H=H, dk=dk, dv=dv, T=T, seed=T)
    x = make_inputs(B, H, dk, dv, T, dtype=torch.bfloat16, seed=T, device=DEV)
    xc = x.to("cpu")
    S_ckpt = x.S0.clone()
    o, rec = run_verify(G, x)
    ref_o = oracle.verify(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta)
    assert rel_err_outputs(o, ref_o) <= OUT_TOL
    assert torch.equal(x.S0, S_ckpt), "verify must not write S"
    n = torch.tensor([0, T, (T + 1) // 2], dtype=torch.int32)
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    G.gdn_commit(x.S0, rec, n.to(DEV), pos)
    ref_S = oracle.commit(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta, n.numpy())
    assert rel_err_state(x.S0, ref_S) <= STATE_TOL
    assert torch.equal(pos.cpu(), n)
    assert torch.equal(x.S0[0].view(torch.int32), S_ckpt[0].view(torch.int32))


def test_slow_decay_and_unit_gate_fixtures(G):
    """g scaled by 0.01 keeps S0's weight near 1 across the block, so errors in the
    state path cannot hide under the decay; g = 0 with beta = 0 must give o = S0 q."""
    B, H, d, T = 2, 4, 128, 8
    print_case(test="slow_decay", B=B, H=H, d=d, T=T, seed=5)
    x = make_inputs(B, H, d, d, T, seed=5, device=DEV, g_scale=0.01, s0_std=1.0)
    xc = x.to("cpu")
    o, rec = run_verify(G, x)
    assert rel_err_outputs(o, oracle.verify(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta)) <= OUT_TOL
    n = torch.tensor([8, 5], dtype=torch.int32)
    G.gdn_commit(x.S0, rec, n.to(DEV))
    ref = oracle.commit(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta, n.numpy())
    assert rel_err_state(x.S0, ref) <= STATE_TOL
    # a = 1, beta = 0.
    y = make_inputs(B, H, d, d, T, seed=6, device=DEV, s0_std=1.0)
    y.g.zero_()
    y.beta.zero_()
    o, rec = run_verify(G, y)
    ref = torch.einsum("bhij,blhj->blhi", y.S0.double().cpu(), y.q.double().cpu())
    assert rel_err_outputs(o, ref) <= 1e-5
    S0 = y.S0.clone()
    G.gdn_commit(y.S0, rec, torch.full((B,), 8, dtype=torch.int32, device=DEV))
    assert rel_err_state(y.S0, S0) <= 1e-6


def test_delta_rule_write_on_gpu(G):
    """a = 1, beta = 1, q_t = k_t: each output is v_t (the write is exact)."""
    B, H, d, T = 1, 4, 128, 8
    print_case(test="delta_write", B=B, H=H, d=d, T=T, seed=9)
    x = make_inputs(B, H, d, d, T, dtype=torch.float32, seed=9, device=DEV)
    x.g.zero_()
    x.beta.fill_(1.0)
    x.q.copy_(x.k)
    o, _ = run_verify(G, x)
    assert rel_err_outputs(o, x.v) <= 1e-4


def test_causality_and_determinism(G):
    B, H, d, T = 2, 8, 128, 8
    print_case(test="causality", B=B, H=H, d=d, T=T, seed=11)
    x = make_inputs(B, H, d, d, T, seed=11, device=DEV)
    o1, _ = run_verify(G, x)
    o2, _ = run_verify(G, x)
    assert torch.equal(o1, o2)
    t = 4
    y = make_inputs(B, H, d, d, T, seed=12, device=DEV)
    for f in ("q", "k", "v", "g", "beta"):
        getattr(x, f)[:, t + 1:] = getattr(y, f)[:, t + 1:]
    o3, _ = run_verify(G, x)
    assert torch.equal(o3[:, : t + 1], o1[:, : t + 1])


def test_commit_error_paths(G):
    B, H, d, T = 2, 4, 64, 8
    print_case(test="commit_errors", B=B, H=H, d=d, T=T, seed=13)
    x = make_inputs(B, H, d, d, T, seed=13, device=DEV)
    S_ckpt = x.S0.clone()
    rec = G.new_record(x.S0, T, x.q.dtype)
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    # Commit before any verify: nothing changes.
    G.gdn_commit(x.S0, rec, torch.tensor([3, 3], dtype=torch.int32, device=DEV), pos)
    assert G.gdn_record_status(rec, x.S0) == [G.GDN_REC_NO_BLOCK] * B
    assert torch.equal(x.S0, S_ckpt) and int(pos.abs().sum()) == 0
    # n out of range for instance 1 only.
    run_verify(G, x, rec)
    G.gdn_commit(x.S0, rec, torch.tensor([2, 9], dtype=torch.int32, device=DEV), pos)
    assert G.gdn_record_status(rec, x.S0) == [0, G.GDN_REC_N_RANGE]
    assert torch.equal(x.S0[1], S_ckpt[1]) and pos.tolist() == [2, 0]
    # Instance 1's block is still pending and commits; instance 0's was consumed.
    G.gdn_commit(x.S0, rec, torch.tensor([2, 4], dtype=torch.int32, device=DEV), pos)
    assert G.gdn_record_status(rec, x.S0) == [G.GDN_REC_NO_BLOCK, G.GDN_REC_N_RANGE]
    assert pos.tolist() == [2, 4]
    xc = x.to("cpu")
    ref = oracle.commit(S_ckpt.cpu(), xc.q, xc.k, xc.v, xc.g, xc.beta, np.array([2, 4], np.int32))
    assert rel_err_state(x.S0, ref) <= STATE_TOL
    # A fresh verify clears the error bits.
    run_verify(G, x, rec)
    assert G.gdn_record_status(rec, x.S0) == [0, 0]
    # Shape mismatch: a record verified with H = 4 committed as H = 2.
    S_small = x.S0[:, :2].contiguous()
    before = S_small.clone()
    G.gdn_commit(S_small, rec, torch.tensor([1, 1], dtype=torch.int32, device=DEV))
    assert torch.equal(S_small, before)
    assert G.gdn_record_status(rec, x.S0) == [G.GDN_REC_SHAPE] * B


def test_speculative_pass_48_layers(G):
    """The 48-layer pass at its real shape: 48 x 32 heads, d = 128, T = 8, bf16,
    then a commit at n ~ U{0..8}; every output and state checked."""
    B, H, d, T = 48, 32, 128, 8
    print_case(test="pass48", B=B, H=H, d=d, T=T, seed=21)
    x = make_inputs(B, H, d, d, T, seed=21, device=DEV)
    xc = x.to("cpu")
    o, rec = run_verify(G, x)
    ref_o = oracle.verify(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta)
    assert rel_err_outputs(o, ref_o) <= OUT_TOL
    n_pass = int(make_accepts(1, T, seed=21)[0])
    n = torch.full((B,), n_pass, dtype=torch.int32)
    n[::7] = torch.arange(len(n[::7]), dtype=torch.int32) % (T + 1)  # a few other n too
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    G.gdn_commit(x.S0, rec, n.to(DEV), pos)
    ref_S = oracle.commit(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta, n.numpy())
    assert rel_err_state(x.S0, ref_S) <= STATE_TOL
    assert torch.equal(pos.cpu(), n)
    zero = (n == 0).nonzero().flatten()
    for b in zero.tolist():
        assert torch.equal(x.S0[b].view(torch.int32), xc.S0[b].to(DEV).view(torch.int32))
