"""GPU parity of gdn_commit_verify: commit the pending block, then verify the
next one, in one pass over the state.

It must equal gdn_commit followed by gdn_verify_block: checked against the
fp64 oracle over chains of speculative passes (outputs of every pass and the
final state, within 2e-3 / 1e-3), against the two separate calls (same bars),
and on every error path of the commit (the state untouched, the same error bits
in the pending record, the new block verified from the unchanged state).
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


def blocks_of(x, T, R):
    """Round r's block: rows r T .. r T + T - 1 of x, contiguous."""
    cut = lambda a, r: a[:, r * T:(r + 1) * T].contiguous()
    return [tuple(cut(getattr(x, f), r) for f in ("q", "k", "v", "g", "beta")) for r in range(R)]


def run_chain(G, S, blocks, ns, T, fused=True):
    """Pass r verifies block r and commits it with ns[r] (device int32 [B]); the
    fused path commits pass r - 1 and verifies pass r in one call."""
    B, H, dv, dk = S.shape
    dt = blocks[0][0].dtype
    recs = [G.new_record(S, T, dt), G.new_record(S, T, dt)]
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    outs = []
    for r, blk in enumerate(blocks):
        o = torch.full((B, T, H, dv), float("nan"), dtype=torch.float32, device=DEV)
        if r == 0 or not fused:
            if r > 0:
                G.gdn_commit(S, recs[(r - 1) % 2], ns[r - 1], pos)
            G.gdn_verify_block(S, *blk, o, recs[r % 2])
        else:
            G.gdn_commit_verify(S, recs[(r - 1) % 2], ns[r - 1], *blk, o, recs[r % 2], pos=pos)
        outs.append(o)
    G.gdn_commit(S, recs[(len(blocks) - 1) % 2], ns[len(blocks) - 1], pos)
    torch.cuda.synchronize()
    return outs, pos, recs


def oracle_chain(S0, blocks, ns):
    S = S0.double().cpu().numpy()
    outs = []
    for blk, n in zip(blocks, ns):
        cpu = [a.cpu() for a in blk]
        outs.append(oracle.verify(S, *cpu))
        S = oracle.commit(S, *cpu, n.cpu().numpy())
    return outs, S


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_fused_chain_matches_oracle(G, dk, dv):
    B, H, T, R = 3, 4, 8, 6
    print_case(test="fused_chain", B=B, H=H, dk=dk, dv=dv, T=T, rounds=R, seed=51)
    x = make_inputs(B, H, dk, dv, T * R, seed=51, device=DEV)
    blocks = blocks_of(x, T, R)
    gen = torch.Generator().manual_seed(52)
    ns = [torch.randint(0, T + 1, (B,), generator=gen, dtype=torch.int32).to(DEV) for _ in range(R)]
    ns[1][:] = T        # a full acceptance and
    ns[2][:] = 0        # a full rollback for every instance
    S = x.S0.clone()
    outs, pos, _ = run_chain(G, S, blocks, ns, T)
    ref_outs, ref_S = oracle_chain(x.S0, blocks, ns)
    for r in range(R):
        assert rel_err_outputs(outs[r], ref_outs[r]) <= OUT_TOL, r
    assert rel_err_state(S, ref_S) <= STATE_TOL
    assert torch.equal(pos, sum(ns))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("T", [1, 3, 8, 12, 16])
@pytest.mark.parametrize("B,H", [(2, 4), (8, 32)], ids=["few_heads", "head_per_wg"])
def test_fused_chain_block_lengths(G, B, H, T, dtype):
    """Chains of fused passes at every block length class (T <= 8 and the
    two-tile form for T = 9 .. 16), fp32 and bf16 block inputs, in both launch
    shapes: fewer than 256 (instance, head) pairs (32 value rows per
    workgroup) and 256 pairs (a head per workgroup)."""
    d, R = 128, 4
    seed = 60 + T + (0 if dtype == torch.bfloat16 else 100) + B
    print_case(test="fused_chain_T", B=B, H=H, d=d, T=T, dtype=dtype, rounds=R, seed=seed)
    x = make_inputs(B, H, d, d, T * R, dtype=dtype, seed=seed, device=DEV)
    blocks = blocks_of(x, T, R)
    gen = torch.Generator().manual_seed(seed)
    ns = [torch.randint(0, T + 1, (B,), generator=gen, dtype=torch.int32).to(DEV) for _ in range(R)]
    ns[1][0] = T
    ns[2][-1] = 0
    S = x.S0.clone()
    outs, pos, _ = run_chain(G, S, blocks, ns, T)
    ref_outs, ref_S = oracle_chain(x.S0, blocks, ns)
    for r in range(R):
        assert rel_err_outputs(outs[r], ref_outs[r]) <= OUT_TOL, r
    assert rel_err_state(S, ref_S) <= STATE_TOL
    assert torch.equal(pos, sum(ns))


def test_fused_equals_separate_calls(G):
    B, H, d, T, R = 4, 8, 128, 8, 5
    print_case(test="fused_vs_separate", B=B, H=H, d=d, T=T, rounds=R, seed=53)
    x = make_inputs(B, H, d, d, T * R, seed=53, device=DEV)
    blocks = blocks_of(x, T, R)
    ns = [torch.full((B,), int(n), dtype=torch.int32, device=DEV) for n in make_accepts(R, T, seed=53)]
    S_f, S_s = x.S0.clone(), x.S0.clone()
    outs_f, pos_f, _ = run_chain(G, S_f, blocks, ns, T, fused=True)
    outs_s, pos_s, _ = run_chain(G, S_s, blocks, ns, T, fused=False)
    for r in range(R):
        assert rel_err_outputs(outs_f[r], outs_s[r]) <= OUT_TOL
    assert rel_err_state(S_f, S_s) <= STATE_TOL
    assert torch.equal(pos_f, pos_s)


def test_fused_zero_accept_leaves_state_bytes(G):
    """n = 0 for an instance: its state is byte-identical after the fused call."""
    B, H, d, T = 2, 4, 128, 8
    print_case(test="fused_zero", B=B, H=H, d=d, T=T, seed=54)
    x = make_inputs(B, H, d, d, 2 * T, seed=54, device=DEV)
    b0, b1 = blocks_of(x, T, 2)
    S = x.S0.clone()
    ra, rb = G.new_record(S, T, torch.bfloat16), G.new_record(S, T, torch.bfloat16)
    o = torch.empty(B, T, H, d, device=DEV)
    G.gdn_verify_block(S, *b0, o, ra)
    G.gdn_commit_verify(S, ra, torch.tensor([0, 5], dtype=torch.int32, device=DEV), *b1, o, rb)
    torch.cuda.synchronize()
    assert torch.equal(S[0].view(torch.int32), x.S0[0].view(torch.int32))
    ref = oracle.commit(x.S0[1:].cpu(), *[a[1:].cpu() for a in b0], np.array([5], np.int32))
    assert rel_err_state(S[1:], ref) <= STATE_TOL
    assert G.gdn_record_status(ra, S) == [0, 0]


def test_fused_long_pending_block_and_fp32_record(G):
    """The pending block has 12 rows (more than the fused path stages at once) and
    fp32 inputs; the next block is bf16."""
    B, H, d = 2, 3, 128
    print_case(test="fused_long_fp32", B=B, H=H, d=d, seed=55)
    x32 = make_inputs(B, H, d, d, 12, dtype=torch.float32, seed=55, device=DEV)
    y = make_inputs(B, H, d, d, 8, seed=56, device=DEV)
    S = x32.S0.clone()
    ra = G.new_record(S, 12, torch.float32)
    rb = G.new_record(S, 8, torch.bfloat16)
    o1 = torch.empty(B, 12, H, d, device=DEV)
    o2 = torch.full((B, 8, H, d), float("nan"), device=DEV)
    G.gdn_verify_block(S, x32.q, x32.k, x32.v, x32.g, x32.beta, o1, ra)
    n = torch.tensor([11, 12], dtype=torch.int32, device=DEV)
    G.gdn_commit_verify(S, ra, n, y.q, y.k, y.v, y.g, y.beta, o2, rb)
    G.gdn_commit(S, rb, torch.tensor([3, 8], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    xc, yc = x32.to("cpu"), y.to("cpu")
    S1 = oracle.commit(xc.S0, xc.q, xc.k, xc.v, xc.g, xc.beta, n.cpu().numpy())
    assert rel_err_outputs(o2, oracle.verify(S1, yc.q, yc.k, yc.v, yc.g, yc.beta)) <= OUT_TOL
    S2 = oracle.commit(S1, yc.q, yc.k, yc.v, yc.g, yc.beta, np.array([3, 8], np.int32))
    assert rel_err_state(S, S2) <= STATE_TOL


def test_fused_error_paths(G):
    B, H, d, T = 2, 4, 64, 8
    print_case(test="fused_errors", B=B, H=H, d=d, T=T, seed=57)
    x = make_inputs(B, H, d, d, 3 * T, seed=57, device=DEV)
    b0, b1, b2 = blocks_of(x, T, 3)
    xc0 = [a.cpu() for a in b0]
    S = x.S0.clone()
    ra, rb = G.new_record(S, T, torch.bfloat16), G.new_record(S, T, torch.bfloat16)
    o = torch.full((B, T, H, d), float("nan"), device=DEV)
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    # Nothing pending in ra: no commit, the new block is verified from S as is.
    G.gdn_commit_verify(S, ra, torch.tensor([3, 3], dtype=torch.int32, device=DEV), *b0, o, rb, pos=pos)
    assert G.gdn_record_status(ra, S) == [G.GDN_REC_NO_BLOCK] * B
    assert torch.equal(S, x.S0) and pos.tolist() == [0, 0]
    assert rel_err_outputs(o, oracle.verify(x.S0.cpu(), *xc0)) <= OUT_TOL
    # rb now holds block 0: n out of range for instance 1 only.
    G.gdn_commit_verify(S, rb, torch.tensor([2, 9], dtype=torch.int32, device=DEV), *b1, o, ra, pos=pos)
    assert G.gdn_record_status(rb, S) == [0, G.GDN_REC_N_RANGE]
    assert torch.equal(S[1], x.S0[1]) and pos.tolist() == [2, 0]
    S_ref = oracle.commit(x.S0.cpu(), *xc0, np.array([2, 0], np.int32))
    assert rel_err_state(S, S_ref) <= STATE_TOL
    assert rel_err_outputs(o, oracle.verify(S_ref, *[a.cpu() for a in b1])) <= OUT_TOL
    # Instance 1's block 0 is still pending in rb; instance 0's was consumed.
    S_before = S.clone()
    G.gdn_commit_verify(S, rb, torch.tensor([2, 4], dtype=torch.int32, device=DEV), *b2, o, ra, pos=pos)
    assert G.gdn_record_status(rb, S) == [G.GDN_REC_NO_BLOCK, G.GDN_REC_N_RANGE]
    assert torch.equal(S[0], S_before[0]) and pos.tolist() == [2, 4]
    S_ref2 = oracle.commit(S_ref[1:], *[a[1:] for a in xc0], np.array([4], np.int32))
    assert rel_err_state(S[1:], S_ref2) <= STATE_TOL
    # Shape mismatch: ra (H = 4) committed with an H = 2 state; nothing changes.
    S_small = S[:, :2].contiguous()
    before = S_small.clone()
    cut = lambda a: a[:, :, :2].contiguous()
    o_small = torch.empty(B, T, 2, d, device=DEV)
    rc_ = G.new_record(S_small, T, torch.bfloat16)
    G.gdn_commit_verify(S_small, ra, torch.tensor([1, 1], dtype=torch.int32, device=DEV),
                        *[cut(a) for a in b0], o_small, rc_)
    assert torch.equal(S_small, before)
    assert G.gdn_record_status(ra, S) == [G.GDN_REC_SHAPE] * B


def test_fused_rejects_same_record(G):
    x = make_inputs(1, 2, 64, 64, 8, seed=58, device=DEV)
    r = G.new_record(x.S0, 8, torch.bfloat16)
    o = torch.empty(1, 8, 2, 64, device=DEV)
    n = torch.ones(1, dtype=torch.int32, device=DEV)
    with pytest.raises(G.GdnError):
        G.gdn_commit_verify(x.S0, r, n, x.q, x.k, x.v, x.g, x.beta, o, r)


def test_fused_48_layers(G):
    """One fused step at the real shape: 48 layers x 32 heads, d = 128, T = 8."""
    B, H, d, T = 48, 32, 128, 8
    print_case(test="fused48", B=B, H=H, d=d, T=T, seed=59)
    x = make_inputs(B, H, d, d, 2 * T, seed=59, device=DEV, device_gen=True)
    b0, b1 = blocks_of(x, T, 2)
    S = x.S0.clone()
    ra, rb = G.new_record(S, T, torch.bfloat16), G.new_record(S, T, torch.bfloat16)
    o0 = torch.empty(B, T, H, d, device=DEV)
    o1 = torch.full((B, T, H, d), float("nan"), device=DEV)
    G.gdn_verify_block(S, *b0, o0, ra)
    n = (torch.arange(B, dtype=torch.int32) % (T + 1)).to(DEV)
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    G.gdn_commit_verify(S, ra, n, *b1, o1, rb, pos=pos)
    torch.cuda.synchronize()
    xc0, xc1 = [a.cpu() for a in b0], [a.cpu() for a in b1]
    S1 = oracle.commit(x.S0.cpu(), *xc0, n.cpu().numpy())
    assert rel_err_state(S, S1) <= STATE_TOL
    assert rel_err_outputs(o1, oracle.verify(S1, *xc1)) <= OUT_TOL
    assert torch.equal(pos.cpu(), n.cpu())
    for b in (n == 0).nonzero().flatten().tolist():
        assert torch.equal(S[b].view(torch.int32), x.S0[b].view(torch.int32))
