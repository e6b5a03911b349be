"""Plain decode (T = 1), chained over 10,000 steps, on both paths.

One GDN layer, 32 heads, d = 128, bf16 q/k/v, fp32 state (2 MiB):
  * the fused path the benchmark times: one gdn_commit_verify per token, which
    commits the previous token (n = 1) and verifies the next (32 heads: the
    few-heads launch, 32 value rows per workgroup);
  * the separate calls: gdn_verify_block on one row, then gdn_commit(n = 1).
Each is checked against the oracle's sequential recurrence over the same
tokens: every output, and the state at steps 1, 10, 100, 1,000 and 10,000.
The transition is non-expansive for a in (0, 1], beta in [0, 2] and |k| <= 1,
so rounding errors must not build up along the chain: the bar at step 10,000
is the same as at step 1.

HIP graphs of the same chained steps must reproduce the eager chains bit for
bit on every replay.
"""
import numpy as np
import pytest
import torch

import oracle
from speculative_verify_amd.inputs import make_inputs
from tests._metrics import OUT_TOL, STATE_TOL, rel_err_outputs, rel_err_state

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def G():
    import speculative_verify_amd.gdn as G
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    return G


def decode_steps(G, x, S, rec, o, t0, t1, one, pos):
    for t in range(t0, t1):
        s = slice(t, t + 1)
        G.gdn_verify_block(S, x.q[:, s], x.k[:, s], x.v[:, s], x.g[:, s], x.beta[:, s], o[:, s], rec)
        G.gdn_commit(S, rec, one, pos)


def fused_steps(G, x, S, recs, o, t0, t1, one, pos):
    """Steps t0 .. t1 - 1 of the fused chain: step t commits token t - 1 (pending
    in recs[(t - 1) % 2]) and verifies token t into recs[t % 2]."""
    for t in range(t0, t1):
        s = slice(t, t + 1)
        G.gdn_commit_verify(S, recs[(t - 1) % 2], one, x.q[:, s], x.k[:, s], x.v[:, s], x.g[:, s], x.beta[:, s],
                            o[:, s], recs[t % 2], pos=pos)


def test_fused_decode_chain_10000_steps(G):
    """The benchmark's decode path, 10,000 chained gdn_commit_verify calls."""
    B, H, d, L = 1, 32, 128, 10000
    print("case: test=fused_decode_chain B=1 H=32 d=128 L=10000 seed=45", flush=True)
    x = make_inputs(B, H, d, d, L, seed=45, device=DEV)
    xc = x.to("cpu")
    S = x.S0.clone()
    recs = [G.new_record(S, 1, torch.bfloat16), G.new_record(S, 1, torch.bfloat16)]
    one = torch.ones(B, dtype=torch.int32, device=DEV)
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    o = torch.full((B, L, H, d), float("nan"), device=DEV)
    G.gdn_verify_block(S, x.q[:, :1], x.k[:, :1], x.v[:, :1], x.g[:, :1], x.beta[:, :1], o[:, :1], recs[0])
    marks = [0, 1, 10, 100, 1000, 10000]
    S_ref = xc.S0.double().numpy()
    for a, b in zip(marks[:-1], marks[1:]):
        # After step t the state holds tokens 0 .. t - 1; the last token is
        # committed by a plain commit.
        if b < L:
            fused_steps(G, x, S, recs, o, a + 1, b + 1, one, pos)
        else:
            fused_steps(G, x, S, recs, o, a + 1, L, one, pos)
            G.gdn_commit(S, recs[(L - 1) % 2], one, pos)
        seg = lambda z: z[:, a:b]
        o_ref, S_ref = oracle.prefill_seq(S_ref, seg(xc.q), seg(xc.k), seg(xc.v), seg(xc.g), seg(xc.beta))
        torch.cuda.synchronize()
        eo, es = rel_err_outputs(o[:, a:b], o_ref), rel_err_state(S, S_ref)
        print(f"  step {b:5d}: out err {eo:.3e}  state err {es:.3e}", flush=True)
        assert eo <= OUT_TOL and es <= STATE_TOL
    assert int(pos[0]) == L
    assert G.gdn_record_status(recs[0], S) == [0] and G.gdn_record_status(recs[1], S) == [0]


def test_fused_decode_graph_replays_match_eager(G):
    """16 chained gdn_commit_verify steps captured in one HIP graph.  Before each
    replay the state, the position and the first token's pending block are
    reset eagerly (with a device sync); every replay must equal the eager chain
    bit for bit."""
    B, H, d, L = 1, 32, 128, 17
    print("case: test=fused_decode_graph B=1 H=32 d=128 L=17 seed=47", flush=True)
    x = make_inputs(B, H, d, d, L, seed=47, device=DEV)
    recs = [G.new_record(x.S0, 1, torch.bfloat16), G.new_record(x.S0, 1, torch.bfloat16)]
    one = torch.ones(B, dtype=torch.int32, device=DEV)
    first = lambda S, o: G.gdn_verify_block(S, x.q[:, :1], x.k[:, :1], x.v[:, :1], x.g[:, :1], x.beta[:, :1],
                                            o[:, :1], recs[0])

    S_e = x.S0.clone()
    pos_e = torch.zeros(B, dtype=torch.int32, device=DEV)
    o_e = torch.empty(B, L, H, d, device=DEV)
    first(S_e, o_e)
    fused_steps(G, x, S_e, recs, o_e, 1, L, one, pos_e)
    torch.cuda.synchronize()

    S = x.S0.clone()
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    o = torch.empty(B, L, H, d, device=DEV)
    first(S, o)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            fused_steps(G, x, S, recs, o, 1, L, one, pos)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        S.copy_(x.S0)
        pos.zero_()
        o.fill_(float("nan"))
        first(S, o)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(S, S_e), f"replay {r}: state differs from the eager chain"
        assert torch.equal(o, o_e), f"replay {r}: outputs differ from the eager chain"
        assert torch.equal(pos, pos_e)


def test_decode_chain_10000_steps(G):
    B, H, d, L = 1, 32, 128, 10000
    print("case: test=decode_chain B=1 H=32 d=128 L=10000 seed=41", flush=True)
    x = make_inputs(B, H, d, d, L, seed=41, device=DEV)
    xc = x.to("cpu")
    S = x.S0.clone()
    rec = G.new_record(S, 1, torch.bfloat16)
    one = torch.ones(B, dtype=torch.int32, device=DEV)
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    o = torch.full((B, L, H, d), float("nan"), device=DEV)
    marks = [0, 1, 10, 100, 1000, 10000]
    S_ref = xc.S0.double().numpy()
    for a, b in zip(marks[:-1], marks[1:]):
        decode_steps(G, x, S, rec, o, a, b, one, pos)
        seg = lambda z: z[:, a:b]
        o_ref, S_ref = oracle.prefill_seq(S_ref, seg(xc.q), seg(xc.k), seg(xc.v), seg(xc.g), seg(xc.beta))
        torch.cuda.synchronize()
        eo, es = rel_err_outputs(o[:, a:b], o_ref), rel_err_state(S, S_ref)
        print(f"  step {b:5d}: out err {eo:.3e}  state err {es:.3e}", flush=True)
        assert eo <= OUT_TOL and es <= STATE_TOL
    assert int(pos[0]) == L
    # The last block was consumed: one more commit changes nothing and says so.
    S_last = S.clone()
    G.gdn_commit(S, rec, one, pos)
    assert G.gdn_record_status(rec, S) == [G.GDN_REC_NO_BLOCK]
    assert torch.equal(S, S_last) and int(pos[0]) == L


def test_decode_graph_replays_match_eager(G):
    """16 chained decode steps captured in one HIP graph.  Each replay starts from
    the same state (reset eagerly between replays, with a device sync) and must
    equal the eager chain bit for bit."""
    B, H, d, L = 1, 32, 128, 16
    print("case: test=decode_graph B=1 H=32 d=128 L=16 seed=43", flush=True)
    x = make_inputs(B, H, d, d, L, seed=43, device=DEV)
    rec = G.new_record(x.S0, 1, torch.bfloat16)
    one = torch.ones(B, dtype=torch.int32, device=DEV)

    S_e = x.S0.clone()
    pos_e = torch.zeros(B, dtype=torch.int32, device=DEV)
    o_e = torch.empty(B, L, H, d, device=DEV)
    decode_steps(G, x, S_e, rec, o_e, 0, L, one, pos_e)
    torch.cuda.synchronize()

    S = x.S0.clone()
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    o = torch.empty(B, L, H, d, device=DEV)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            decode_steps(G, x, S, rec, o, 0, L, one, pos)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        S.copy_(x.S0)
        pos.zero_()
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(S, S_e), f"replay {r}: state differs from the eager chain"
        assert torch.equal(o, o_e), f"replay {r}: outputs differ from the eager chain"
        assert torch.equal(pos, pos_e)
