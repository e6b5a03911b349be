"""GPU parity of gdn_prefill_chunked against the fp64 sequential oracle.

Bars: outputs within 2e-3 and the final state within 1e-3 (worst (instance,
head) slab, max|x - r| / max|r|).  The chunk form must reach the token-by-token
result: the oracle here is the sequential recurrence, not a chunked one.
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


def print_case(**kw):
    print("case:", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def run_prefill(G, x):
    B, H, dk, dv, L = x.shape
    o = torch.full((B, L, H, dv), float("nan"), dtype=torch.float32, device=DEV)
    S = x.S0.clone()
    G.gdn_prefill_chunked(S, x.q, x.k, x.v, x.g, x.beta, o)
    torch.cuda.synchronize()
    return o, S


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("L", [1, 64, 65, 200])
def test_prefill_shapes_and_tails(G, dk, dv, L):
    B, H = 2, 3
    print_case(test="prefill_shapes", B=B, H=H, dk=dk, dv=dv, L=L, seed=L)
    x = make_inputs(B, H, dk, dv, L, seed=L, device=DEV)
    xc = x.to("cpu")
    o, S = run_prefill(G, x)
    ref_o, ref_S = oracle.prefill_seq(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta)
    assert not torch.isnan(o).any()
    assert rel_err_outputs(o, ref_o) <= OUT_TOL
    assert rel_err_state(S, ref_S) <= STATE_TOL


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64)])
def test_prefill_segmented_schedule_ragged(G, dk, dv):
    """Few heads and enough chunks (17, the last partial) that the two-phase
    schedule cuts the prompt into segments, each segment's prep running beside
    the previous segment's scan: every output and the final state against the
    sequential oracle."""
    B, H, L = 1, 3, 16 * 64 + 37
    print_case(test="prefill_segmented", B=B, H=H, dk=dk, dv=dv, L=L, seed=57)
    x = make_inputs(B, H, dk, dv, L, seed=57, device=DEV)
    xc = x.to("cpu")
    o, S = run_prefill(G, x)
    ref_o, ref_S = oracle.prefill_seq(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta)
    assert not torch.isnan(o).any()
    eo, es = rel_err_outputs(o, ref_o), rel_err_state(S, ref_S)
    print(f"prefill_segmented: out err {eo:.3e} state err {es:.3e}", flush=True)
    assert eo <= OUT_TOL and es <= STATE_TOL


def test_prefill_4096_tokens_32_heads(G):
    """One layer, 32 heads, d = 128, 4,096 tokens, chunk 64: every output and the
    final state against the sequential oracle."""
    B, H, d, L = 1, 32, 128, 4096
    print_case(test="prefill_4096", B=B, H=H, d=d, L=L, seed=3)
    x = make_inputs(B, H, d, d, L, seed=3, device=DEV)
    xc = x.to("cpu")
    o, S = run_prefill(G, x)
    ref_o, ref_S = oracle.prefill_seq(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta)
    eo, es = rel_err_outputs(o, ref_o), rel_err_state(S, ref_S)
    print(f"prefill_4096: out err {eo:.3e} state err {es:.3e}", flush=True)
    assert eo <= OUT_TOL and es <= STATE_TOL


def test_prefill_slow_decay(G):
    """g scaled by 0.01: the state keeps most of its history across chunks, so
    inter-chunk errors cannot hide under the decay."""
    B, H, d, L = 1, 8, 128, 1000
    print_case(test="prefill_slow_decay", B=B, H=H, d=d, L=L, seed=4)
    x = make_inputs(B, H, d, d, L, seed=4, device=DEV, g_scale=0.01, s0_std=1.0)
    xc = x.to("cpu")
    o, S = run_prefill(G, x)
    ref_o, ref_S = oracle.prefill_seq(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta)
    assert rel_err_outputs(o, ref_o) <= OUT_TOL
    assert rel_err_state(S, ref_S) <= STATE_TOL


def test_prefill_split_prompt_and_empty(G):
    """prefill(L1) then prefill(L2) on the continued inputs equals prefill(L1 + L2)
    within the bars; L = 0 changes nothing."""
    B, H, d, L, cut = 2, 4, 128, 300, 100
    print_case(test="prefill_split", B=B, H=H, d=d, L=L, seed=5)
    x = make_inputs(B, H, d, d, L, seed=5, device=DEV)
    o_full, S_full = run_prefill(G, x)
    part = lambda a, sl: a[:, sl].contiguous()
    S = x.S0.clone()
    o1 = torch.empty(B, cut, H, d, device=DEV)
    o2 = torch.empty(B, L - cut, H, d, device=DEV)
    a, z = slice(0, cut), slice(cut, L)
    G.gdn_prefill_chunked(S, part(x.q, a), part(x.k, a), part(x.v, a), part(x.g, a), part(x.beta, a), o1)
    G.gdn_prefill_chunked(S, part(x.q, z), part(x.k, z), part(x.v, z), part(x.g, z), part(x.beta, z), o2)
    torch.cuda.synchronize()
    assert rel_err_outputs(torch.cat([o1, o2], 1), o_full) <= OUT_TOL
    assert rel_err_state(S, S_full) <= STATE_TOL
    S0 = S.clone()
    e = torch.empty(B, 0, H, d, device=DEV)
    G.gdn_prefill_chunked(S, x.q[:, :0], x.k[:, :0], x.v[:, :0], x.g[:, :0], x.beta[:, :0], e)
    torch.cuda.synchronize()
    assert torch.equal(S, S0)


def test_verify_commit_equals_prefill(G):
    """verify + commit(T) of a block = prefill of the same T tokens (outputs and
    state), two independent kernels reaching the same definition."""
    B, H, d, T = 3, 8, 128, 8
    print_case(test="verify_vs_prefill", B=B, H=H, d=d, T=T, seed=6)
    x = make_inputs(B, H, d, d, T, seed=6, device=DEV)
    o_p, S_p = run_prefill(G, x)
    o_v = torch.empty_like(o_p)
    rec = G.new_record(x.S0, T, x.q.dtype)
    S_v = x.S0.clone()
    G.gdn_verify_block(S_v, x.q, x.k, x.v, x.g, x.beta, o_v, rec)
    G.gdn_commit(S_v, rec, torch.full((B,), T, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    assert rel_err_outputs(o_v, o_p) <= OUT_TOL
    assert rel_err_state(S_v, S_p) <= STATE_TOL


def test_prefill_rejects_fp32_inputs(G):
    x = make_inputs(1, 2, 64, 64, 8, dtype=torch.float32, seed=7, device=DEV)
    o = torch.empty(1, 8, 2, 64, device=DEV)
    with pytest.raises(G.GdnError):
        G.gdn_prefill_chunked(x.S0, x.q, x.k, x.v, x.g, x.beta, o)


def test_prefill_48_layers_32k_then_256_rounds(G):
    """Long context: 48 layers x 32 heads, d = 128, a 32,768-token prompt in one
    launch, then 256 speculative rounds (T = 8 verify, commit at n ~ U{0..8},
    one n per round for all layers) on the prefilled state.  Sampled (layer,
    head) pairs against the oracle: the prompt's outputs and final state, every
    round's outputs, and the state after the last round."""
    B, H, d, L, T, R = 48, 32, 128, 32768, 8, 256
    print_case(test="prefill_48x32k_rounds", B=B, H=H, d=d, L=L, rounds=R, seed=8)
    x = make_inputs(B, H, d, d, L, seed=8, device=DEV, device_gen=True)
    o = torch.empty(B, L, H, d, dtype=torch.float32, device=DEV)
    S = x.S0.clone()
    G.gdn_prefill_chunked(S, x.q, x.k, x.v, x.g, x.beta, o)
    torch.cuda.synchronize()
    picks = [(0, 0), (17, 31), (47, 5)]
    ref_state = {}
    for (b, h) in picks:
        pick = lambda a: a[b:b + 1, :, h:h + 1].contiguous().cpu()
        ref_o, ref_S = oracle.prefill_seq(x.S0[b:b + 1, h:h + 1].cpu(), pick(x.q), pick(x.k),
                                          pick(x.v), pick(x.g), pick(x.beta))
        eo = rel_err_outputs(o[b:b + 1, :, h:h + 1], ref_o)
        es = rel_err_state(S[b:b + 1, h:h + 1], ref_S)
        print(f"  prefill (b={b}, h={h}): out {eo:.3e} state {es:.3e}", flush=True)
        assert eo <= OUT_TOL and es <= STATE_TOL
        ref_state[(b, h)] = ref_S
    del x, o
    torch.cuda.empty_cache()

    # 256 rounds on the prefilled state.
    y = make_inputs(B, H, d, d, R * T, seed=9, device=DEV, device_gen=True)
    ns = make_accepts(R, T, seed=9)
    rec = G.new_record(S, T, torch.bfloat16)
    ob = torch.empty(B, T, H, d, dtype=torch.float32, device=DEV)
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    got = {p: [] for p in picks}
    for r in range(R):
        blk = lambda a: a[:, r * T:(r + 1) * T].contiguous()
        G.gdn_verify_block(S, blk(y.q), blk(y.k), blk(y.v), blk(y.g), blk(y.beta), ob, rec)
        G.gdn_commit(S, rec, torch.full((B,), int(ns[r]), dtype=torch.int32, device=DEV), pos)
        for (b, h) in picks:
            got[(b, h)].append(ob[b:b + 1, :, h:h + 1].cpu())
    torch.cuda.synchronize()
    assert pos.tolist() == [int(ns.sum())] * B
    for (b, h) in picks:
        S_ref, worst = ref_state[(b, h)], 0.0
        for r in range(R):
            blk = lambda a: a[b:b + 1, r * T:(r + 1) * T, h:h + 1].contiguous().cpu()
            args = (blk(y.q), blk(y.k), blk(y.v), blk(y.g), blk(y.beta))
            worst = max(worst, rel_err_outputs(got[(b, h)][r], oracle.verify(S_ref, *args)))
            S_ref = oracle.commit(S_ref, *args, np.array([int(ns[r])], np.int32))
        es = rel_err_state(S[b:b + 1, h:h + 1], S_ref)
        print(f"  rounds (b={b}, h={h}): worst round out {worst:.3e} final state {es:.3e}", flush=True)
        assert worst <= OUT_TOL and es <= STATE_TOL
    del y, S
    torch.cuda.empty_cache()


@pytest.mark.parametrize("schedule", ["two_pass", "one_pass"])
@pytest.mark.parametrize("dk,dv,L", [(128, 128, 300), (64, 128, 129), (128, 64, 64)])
def test_prefill_both_schedules(G, schedule, dk, dv, L):
    """Few heads run two phases (parallel chunk prep into the workspace, and the
    scan) when given the workspace, and one pass without it; both reach the
    sequential oracle."""
    B, H = 1, 4
    print_case(test="prefill_schedules", schedule=schedule, dk=dk, dv=dv, L=L, seed=31)
    x = make_inputs(B, H, dk, dv, L, seed=31, device=DEV)
    xc = x.to("cpu")
    need = G.gdn_prefill_workspace_bytes(x.S0, L)
    assert need > 0
    ws = torch.empty(need if schedule == "two_pass" else 0, dtype=torch.uint8, device=DEV)
    o = torch.full((B, L, H, dv), float("nan"), dtype=torch.float32, device=DEV)
    S = x.S0.clone()
    G.gdn_prefill_chunked(S, x.q, x.k, x.v, x.g, x.beta, o, ws=ws)
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.prefill_seq(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta)
    assert not torch.isnan(o).any()
    assert rel_err_outputs(o, ref_o) <= OUT_TOL
    assert rel_err_state(S, ref_S) <= STATE_TOL


@pytest.mark.parametrize("dk", [128, 64])
@pytest.mark.parametrize("L", [1, 64, 65, 200])
def test_prefill_one_pass_many_heads(G, dk, L):
    """256 (instance, head) pairs take the one-pass kernel (a workgroup per head,
    two heads per compute unit): every output and the final state against the
    sequential oracle, with full and partial last chunks."""
    B, H, dv = 8, 32, 128
    print_case(test="prefill_one_pass_many", B=B, H=H, dk=dk, dv=dv, L=L, seed=41 + L)
    x = make_inputs(B, H, dk, dv, L, seed=41 + L, device=DEV)
    xc = x.to("cpu")
    assert G.gdn_prefill_workspace_bytes(x.S0, L) == 0
    o = torch.full((B, L, H, dv), float("nan"), dtype=torch.float32, device=DEV)
    S = x.S0.clone()
    G.gdn_prefill_chunked(S, x.q, x.k, x.v, x.g, x.beta, o)
    torch.cuda.synchronize()
    ref_o, ref_S = oracle.prefill_seq(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta)
    assert not torch.isnan(o).any()
    assert rel_err_outputs(o, ref_o) <= OUT_TOL
    assert rel_err_state(S, ref_S) <= STATE_TOL
