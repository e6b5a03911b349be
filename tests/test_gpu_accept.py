"""GPU parity of on-device acceptance and rewind against the fp64 oracle
(oracle/accept_oracle.py), through libgdn's C ABI.

Bars:
  * greedy: n and the emitted token bit-exact (argmax of the exact logits, the
    lowest index among equals, on both sides);
  * sampled: every sequence's (n, token) is the oracle's outcome.  Where a keep
    decision lies within fp32 rounding of its threshold (|u q - p| / max(p, q)
    < 1e-4) either way is correct, so the outcome must be the oracle's on one
    of the branches those decisions open (the oracle takes them the other way
    on request): the decisions before the first such one match exactly, and n
    and the token are one branch's.  Where the draw itself lies within fp32
    rounding of a cumulative boundary (u * total within 2e-5 of the total),
    the token must be a valid draw: its fp64 cumulative interval contains
    u * total within that band, and its weight is not negative.  The band must
    hold few cases;
  * rewind: bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import accept_oracle as A
from speculative_verify_amd.inputs import make_accept_inputs, make_history_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ACC_BAND, DRAW_BAND = 1e-4, 2e-5
VQ = 151936   # the Qwen3 tokenizer's vocabulary size


@pytest.fixture(scope="module")
def G():
    import speculative_verify_amd.gdn as G
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    return G


def print_case(**kw):
    print("case:", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def run_greedy(G, x):
    B = x.target.shape[0]
    n = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    nxt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    G.gdn_accept_greedy(x.target, x.tokens, n, nxt)
    torch.cuda.synchronize()
    return n.cpu().numpy(), nxt.cpu().numpy()


def run_sampled(G, x, tau):
    B = x.target.shape[0]
    n = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    nxt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    G.gdn_accept_sampled(x.target, x.draft, x.tokens, x.u_accept, x.u_sample, tau, n, nxt)
    torch.cuda.synchronize()
    return n.cpu().numpy(), nxt.cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("T,V", [(1, 1000), (2, 4097), (8, VQ), (16, 1000), (8, 1), (8, 4096)])
def test_greedy_matches_oracle(G, T, V, dtype):
    B = 48
    print_case(test="accept_greedy", B=B, T=T, V=V, dtype=dtype, seed=T * 1000 + V)
    x = make_accept_inputs(B, T, V, dtype=dtype, seed=T * 1000 + V, device=DEV, plan_greedy=True)
    n, nxt = run_greedy(G, x)
    xc = x.to("cpu")
    rn, rx = A.accept_greedy(xc.target.float().numpy(), xc.tokens.numpy())
    assert np.array_equal(n, rn), (n, rn)
    assert np.array_equal(nxt, rx), (nxt, rx)
    if V > 1 and T > 1:
        assert len(set(n.tolist())) > 1   # the plan spreads the accepted lengths


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_greedy_ties_take_the_lowest_index(G, dtype):
    """Logits quantised to a few levels: every row has many tied maxima."""
    B, T, V = 32, 8, 5000
    print_case(test="accept_greedy_ties", B=B, T=T, V=V, dtype=dtype, seed=11)
    gen = torch.Generator().manual_seed(11)
    z = torch.randint(0, 4, (B, T, V), generator=gen).to(torch.float32).to(dtype)
    first = (z == 3).float().argmax(dim=2)            # lowest index of the top level
    k = torch.randint(0, T, (B,), generator=gen)
    d = first[:, : T - 1].clone().to(torch.int32)
    for b in range(B):                                 # keep k drafts, then a tied-but-later index
        if int(k[b]) < T - 1:
            j = int(k[b])
            later = torch.nonzero(z[b, j] == 3).flatten()
            d[b, j] = int(later[-1]) if len(later) > 1 else (int(first[b, j]) + 1) % V
    from speculative_verify_amd.inputs import AcceptInputs
    x = AcceptInputs(z.to(DEV), z[:, : T - 1].contiguous().to(DEV), d.to(DEV),
                     torch.zeros(B, T - 1, device=DEV), torch.zeros(B, device=DEV))
    n, nxt = run_greedy(G, x)
    rn, rx = A.accept_greedy(z.float().numpy(), d.numpy())
    assert np.array_equal(n, rn) and np.array_equal(nxt, rx)


def branches(z, y, d, ua, us, tau, b):
    """Every outcome of sequence b that fp32 rounding can reach: the oracle's own
    path, and the paths with any of its near-threshold keep decisions (margin
    below ACC_BAND) taken the other way, followed to their ends (each flipped
    path is explored for further near-threshold decisions, up to three flips).
    Returns [(n, token, info)]."""
    out, seen, todo = [], set(), [frozenset()]
    while todo:
        fl = todo.pop()
        if fl in seen:
            continue
        seen.add(fl)
        rn, rx, info = A.accept_sampled(z[b:b + 1], y[b:b + 1], d[b:b + 1], ua[b:b + 1], us[b:b + 1], tau,
                                        flip={0: set(fl)})
        out.append((int(rn[0]), int(rx[0]), info[0]))
        if len(fl) < 3:
            for j, mg in enumerate(info[0]["accept_margins"]):
                if mg < ACC_BAND and j not in fl:
                    todo.append(fl | {j})
    return out


def valid_draw(w, u, x_):
    """The kernel's token x_ is a draw from weights w at uniform u up to fp32
    rounding: its fp64 cumulative interval contains u * total within DRAW_BAND of
    the total, and its weight is not negative."""
    c = np.cumsum(w)
    t = float(u) * c[-1]
    if not 0 <= x_ < len(w):
        return False
    lo = c[x_ - 1] if x_ > 0 else 0.0
    return lo <= t + DRAW_BAND * c[-1] and c[x_] >= t - DRAW_BAND * c[-1] and w[x_] >= -1e-6 * w.max()


def check_sampled(x, tau, n, nxt):
    """Every sequence: the kernel's (n, token) is the oracle's outcome on one of
    the branches fp32 rounding can reach (its own path when every decision is
    clear of its threshold).  On that branch the token must equal the oracle's
    where the draw is clear of the cumulative boundaries, and be a valid draw
    where it is not.  Returns (sequences on the oracle's path with a clear
    draw, sequences that needed the band)."""
    xc = x.to("cpu")
    z, y = xc.target.float().numpy(), xc.draft.float().numpy()
    d, ua, us = xc.tokens.numpy(), xc.u_accept.numpy(), xc.u_sample.numpy()
    rn, rx, info = A.accept_sampled(z, y, d, ua, us, tau)
    clear = band = 0
    B, T, _ = z.shape
    for b in range(B):
        near = min(info[b]["accept_margins"], default=1.0) < ACC_BAND
        paths = branches(z, y, d, ua, us, tau, b) if near else [(int(rn[b]), int(rx[b]), info[b])]
        ok = False
        for pn, px, pinfo in paths:
            if n[b] != pn:
                continue
            m = pinfo["m"]
            p = A.softmax(z[b, m], tau)
            w = np.maximum(p - A.softmax(y[b, m], tau), 0.0) if pinfo["kind"] == "correction" else p
            exact = pinfo["draw_margin"] >= DRAW_BAND
            if (exact and int(nxt[b]) == px) or (not exact and valid_draw(w, us[b], int(nxt[b]))):
                ok = True
                break
        assert ok, (b, int(n[b]), int(nxt[b]), [(pn, px) for pn, px, _ in paths], info[b])
        if not near and info[b]["draw_margin"] >= DRAW_BAND:
            clear += 1
        else:
            band += 1
    return clear, band


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("T,V,tau,peak", [(8, VQ, 1.0, 16.0), (8, 1000, 0.7, 8.0), (16, 4096, 1.3, 12.0),
                                          (1, 5000, 1.0, 12.0), (2, 3, 1.0, 0.0), (8, VQ, 1.0, 0.0)])
def test_sampled_matches_oracle(G, T, V, tau, peak, dtype):
    """Peaked rows (a few likely tokens over the tail) put the draws clear of
    fp32 rounding, where the token must be exact; the last case, flat rows over
    151,936 entries, puts nearly every draw within rounding of a cumulative
    boundary, where only validity is required."""
    B = 64
    seed = 7 * T + V
    print_case(test="accept_sampled", B=B, T=T, V=V, tau=tau, peak=peak, dtype=dtype, seed=seed)
    x = make_accept_inputs(B, T, V, dtype=dtype, seed=seed, device=DEV, tau=tau, peak=peak)
    n, nxt = run_sampled(G, x, tau)
    clear, band = check_sampled(x, tau, n, nxt)
    print(f"  clear {clear}, in the rounding band {band}", flush=True)
    flat = peak == 0.0 and V > 1000
    if not flat:
        assert band <= max(2, B // 8)
    if T > 1 and V > 3:
        assert len(set(n.tolist())) > 1


def test_sampled_single_entry_vocabulary(G):
    """V = 1: p = q = 1, every draft is kept and the bonus is token 0."""
    B, T = 4, 8
    x = make_accept_inputs(B, T, 1, dtype=torch.float32, seed=3, device=DEV)
    n, nxt = run_sampled(G, x, 1.0)
    assert (n == T).all() and (nxt == 0).all()


def test_out_of_range_drafts_are_rejected(G):
    B, T, V = 4, 8, 1000
    x = make_accept_inputs(B, T, V, dtype=torch.float32, seed=5, device=DEV, drift=0.0)
    x.tokens[:, 0] = torch.tensor([-1, V, 1 << 30, -(1 << 30)], dtype=torch.int32, device=DEV)
    n, _ = run_sampled(G, x, 1.0)
    assert (n == 1).all()
    ng, _ = run_greedy(G, x)
    assert (ng == 1).all()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("W,C", [(1, 1), (3, 300), (4, 8192), (16, 257)])
def test_history_rewind_matches_oracle(G, W, C, dtype):
    B, T = 3, 8
    for ns in ([0, 1, T], [T - 1, 2, 3], [-1, T + 1, 5]):
        print_case(test="history_rewind", B=B, W=W, T=T, C=C, dtype=dtype, n=ns)
        hist, rows = make_history_inputs(B, W, T, C, dtype=dtype, seed=W * C, device=DEV)
        h0 = hist.clone()
        n = torch.tensor(ns, dtype=torch.int32, device=DEV)
        G.gdn_history_rewind(hist, rows, n)
        torch.cuda.synchronize()
        for b in range(B):
            if 0 <= ns[b] <= T:
                ref = A.conv_window_rewind(h0[b:b + 1].cpu().float().numpy(), rows[b:b + 1].cpu().float().numpy(),
                                           np.array([ns[b]]))[0]
                assert np.array_equal(hist[b].cpu().float().numpy(), ref), (b, ns[b])
            else:   # out of range: unchanged
                assert torch.equal(hist[b], h0[b])


def test_accept_feeds_commit_on_the_device(G):
    """The GPU-resident loop: verify a block, accept it greedily against planted
    target logits, commit the device-side n; three passes, no host round trip in
    between.  The state must equal the oracle's commit of the same n values."""
    from speculative_verify_amd.inputs import make_inputs
    B, H, d, T, V, P = 1, 4, 64, 8, 1000, 3
    print_case(test="accept_commit_loop", B=B, H=H, d=d, T=T, V=V, passes=P, seed=77)
    x = make_inputs(B, H, d, d, P * T, seed=77, device=DEV)
    acc = make_accept_inputs(P, T, V, dtype=torch.bfloat16, seed=77, device=DEV, plan_greedy=True)
    S = x.S0.clone()
    rec = G.new_record(S, T, x.q.dtype)
    pos = torch.zeros(B, dtype=torch.int32, device=DEV)
    o = torch.empty(B, T, H, d, device=DEV)
    n = torch.empty(B, dtype=torch.int32, device=DEV)
    nxt = torch.empty(B, dtype=torch.int32, device=DEV)
    blk = lambda t, r: tuple(getattr(t, f)[:, r * T:(r + 1) * T].contiguous() for f in ("q", "k", "v", "g", "beta"))
    for r in range(P):
        G.gdn_verify_block(S, *blk(x, r), o, rec)
        G.gdn_accept_greedy(acc.target[r:r + 1].contiguous(), acc.tokens[r:r + 1].contiguous(), n, nxt)
        G.gdn_commit(S, rec, n, pos)
    torch.cuda.synchronize()
    xc, ac = x.to("cpu"), acc.to("cpu")
    rn, _ = A.accept_greedy(ac.target.float().numpy(), ac.tokens.numpy())
    S_ref = xc.S0.double().numpy()
    for r in range(P):
        S_ref = oracle.commit(S_ref, *blk(xc, r), np.array([rn[r]], np.int32))
    from tests._metrics import STATE_TOL, rel_err_state
    assert int(pos[0]) == int(rn.sum())
    assert rel_err_state(S, S_ref) <= STATE_TOL
