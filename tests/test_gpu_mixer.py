"""GPU parity of the verify with the GDN mixer fused around it
(gdn_mixer_verify, gdn_mixer_commit_verify) against the fp64 oracles: the mixer
prologue and epilogue of oracle/mixer_oracle.py around the recurrence of the C
oracle.  Bars: outputs within 2e-3 and committed state within 1e-3 (worst-slab
relative, as for the verify).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import mixer_oracle as M
from speculative_verify_amd.inputs import make_inputs, make_mixer_inputs
from tests._metrics import OUT_TOL, STATE_TOL, rel_err_outputs, rel_err_state

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
D = 128


@pytest.fixture(scope="module")
def G():
    import speculative_verify_amd.gdn as G
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    return G


def print_case(**kw):
    print("case:", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def ref_block(S0, mc, H):
    """Oracle: prologue, verify outputs and the gated norm; the prologue's q, k,
    v, g, beta returned for the commit."""
    f = lambda t: t.float().numpy()
    q, k, v, g, beta = M.prologue(f(mc.x), f(mc.history), f(mc.conv_w), f(mc.a), f(mc.b), f(mc.A_log),
                                  f(mc.dt_bias), mc.Hk, D, H, D)
    o = oracle.verify(S0, q, k, v, g, beta)
    return M.epilogue(o, f(mc.z), f(mc.norm_w)), (q, k, v, g, beta)


@pytest.mark.parametrize("B,H,Hk,T", [(2, 4, 2, 8), (1, 32, 16, 8), (2, 4, 4, 1), (1, 8, 2, 12)])
def test_mixer_verify_then_commit(G, B, H, Hk, T):
    print_case(test="mixer_verify", B=B, H=H, Hk=Hk, T=T, seed=B * 100 + H + T)
    S0 = make_inputs(B, H, D, D, 1, seed=B * 100 + H + T, device=DEV).S0
    m = make_mixer_inputs(B, T, H, Hk, D, seed=B * 100 + H + T, device=DEV)
    y = torch.full((B, T, H, D), float("nan"), device=DEV)
    S = S0.clone()
    rec = G.new_record(S, T, torch.bfloat16)
    G.gdn_mixer_verify(S, m, y, rec)
    n = torch.tensor([(3 * b + 2) % (T + 1) for b in range(B)], dtype=torch.int32, device=DEV)
    G.gdn_commit(S, rec, n)
    torch.cuda.synchronize()
    S0c = S0.cpu().double().numpy()
    y_ref, qkv = ref_block(S0c, m.to("cpu"), H)
    eo = rel_err_outputs(y, y_ref)
    es = rel_err_state(S, oracle.commit(S0c, *qkv, n.cpu().numpy()))
    print(f"  output err {eo:.2e} state err {es:.2e}", flush=True)
    assert eo <= OUT_TOL and es <= STATE_TOL


@pytest.mark.parametrize("T,n0,n1", [(8, 5, 3), (12, 10, 7), (16, 16, 9), (1, 1, 0)])
def test_mixer_commit_verify_two_blocks(G, T, n0, n1):
    """Block 0 by gdn_mixer_verify, then block 1 by gdn_mixer_commit_verify at
    n = n0: the outputs of block 1 come from S_n0 of block 0, and a final commit
    of block 1 at n = n1 lands on the oracle's state.  Blocks longer than 8 rows
    replay their rows past the eighth straight from the record."""
    B, H, Hk = 2, 8, 4
    print_case(test="mixer_commit_verify", B=B, H=H, Hk=Hk, T=T, n0=n0, n1=n1, seed=21 + T)
    S0 = make_inputs(B, H, D, D, 1, seed=21 + T, device=DEV).S0
    full = make_mixer_inputs(B, 2 * T, H, Hk, D, seed=21 + T, device=DEV)
    m0, m1 = full.block(0, T), full.block(1, T)
    S = S0.clone()
    ra, rb = G.new_record(S, T, torch.bfloat16), G.new_record(S, T, torch.bfloat16)
    y0 = torch.empty(B, T, H, D, device=DEV)
    y1 = torch.empty(B, T, H, D, device=DEV)
    G.gdn_mixer_verify(S, m0, y0, ra)
    G.gdn_mixer_commit_verify(S, ra, torch.full((B,), n0, dtype=torch.int32, device=DEV), m1, y1, rb)
    G.gdn_commit(S, rb, torch.full((B,), n1, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    S0c = S0.cpu().double().numpy()
    y0_ref, qkv0 = ref_block(S0c, m0.to("cpu"), H)
    Sn = oracle.commit(S0c, *qkv0, np.full(B, n0, np.int32))
    y1_ref, qkv1 = ref_block(Sn, m1.to("cpu"), H)
    S_ref = oracle.commit(Sn, *qkv1, np.full(B, n1, np.int32))
    e0, e1, es = rel_err_outputs(y0, y0_ref), rel_err_outputs(y1, y1_ref), rel_err_state(S, S_ref)
    print(f"  outputs {e0:.2e} / {e1:.2e}, state {es:.2e}", flush=True)
    assert e0 <= OUT_TOL and e1 <= OUT_TOL and es <= STATE_TOL


def test_mixer_48_layers_sampled(G):
    """The benchmark's shape and launch: 48 layers x 32 value heads (16 q/k heads),
    T = 8, a mixer verify, then a fused commit (n = 5) + mixer verify of the next
    block.  Layers 0, 23 and 47 against the oracle computed for them alone."""
    B, H, Hk, T = 48, 32, 16, 8
    print_case(test="mixer_48_layers", B=B, H=H, Hk=Hk, T=T, seed=31)
    S0 = make_inputs(B, H, D, D, 1, seed=31, device=DEV, device_gen=True).S0
    full = make_mixer_inputs(B, 2 * T, H, Hk, D, seed=31, device=DEV)
    m0, m1 = full.block(0, T), full.block(1, T)
    S = S0.clone()
    ra, rb = G.new_record(S, T, torch.bfloat16), G.new_record(S, T, torch.bfloat16)
    y0 = torch.empty(B, T, H, D, device=DEV)
    y1 = torch.empty(B, T, H, D, device=DEV)
    G.gdn_mixer_verify(S, m0, y0, ra)
    G.gdn_mixer_commit_verify(S, ra, torch.full((B,), 5, dtype=torch.int32, device=DEV), m1, y1, rb)
    torch.cuda.synchronize()

    def layer(m, b):
        pick = lambda t: t[b:b + 1].contiguous()
        return type(m)(pick(m.x), pick(m.history), m.conv_w, pick(m.a), pick(m.b), m.A_log, m.dt_bias,
                       pick(m.z), m.norm_w, m.Hk).to("cpu")

    for b in (0, 23, 47):
        S0b = S0[b:b + 1].cpu().double().numpy()
        y0_ref, qkv0 = ref_block(S0b, layer(m0, b), H)
        S5 = oracle.commit(S0b, *qkv0, np.array([5], np.int32))
        y1_ref, _ = ref_block(S5, layer(m1, b), H)
        e0, e1 = rel_err_outputs(y0[b:b + 1], y0_ref), rel_err_outputs(y1[b:b + 1], y1_ref)
        es = rel_err_state(S[b:b + 1], S5)
        print(f"  layer {b}: out {e0:.2e} / {e1:.2e}, state {es:.2e}", flush=True)
        assert e0 <= OUT_TOL and e1 <= OUT_TOL and es <= STATE_TOL
