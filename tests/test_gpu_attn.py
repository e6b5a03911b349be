"""GPU parity of the verify pass's full-attention mixer (gdn_attn_verify)
against the fp64 oracle (oracle/attn_oracle.py), through libgdn's C ABI.

Bar: |o - ref| <= 4e-3 * max|v| per output, written out below.  The arithmetic
it follows from: q, k, v enter exactly (bf16); scores and the running softmax
are fp32; the attention weights enter the P V product as bf16, a relative
rounding of at most 2^-9 on each weight, so an output (a weighted average of
values) moves by at most about 2^-8 max|v| even if every rounding had the same
sign.  The cache append is bit-exact.
"""
import numpy as np
import pytest
import torch

from oracle import attn_oracle as A
from speculative_verify_amd.inputs import make_attn_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 4e-3


@pytest.fixture(scope="module")
def G():
    import speculative_verify_amd.gdn as G
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    return G


def print_case(**kw):
    print("case:", " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def run(G, x, scale=None):
    B, T, Hq, d = x.q.shape
    o = torch.full((B, T, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    kc, vc = x.k_cache.clone(), x.v_cache.clone()
    G.gdn_attn_verify(x.q, x.k_new, x.v_new, kc, vc, x.ctx, o, scale=scale)
    torch.cuda.synchronize()
    return o, kc, vc


def check(x, o, kc, vc, scale):
    xc = x.to("cpu")
    f = lambda t: t.float().numpy()
    ref, rk, rv = A.attn_verify(f(xc.q), f(xc.k_new), f(xc.v_new), f(xc.k_cache), f(xc.v_cache), xc.ctx.numpy(),
                                scale)
    vmax = max(float(xc.v_cache.float().abs().max()), float(xc.v_new.float().abs().max()))
    err = np.abs(o.cpu().double().numpy() - ref).max()
    assert err <= TOL * vmax, (err, vmax)
    # The block's rows are in the cache; every other cache row is untouched.
    assert np.array_equal(kc.cpu().float().numpy(), rk)
    assert np.array_equal(vc.cpu().float().numpy(), rv)
    return err / vmax


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("T,Hq,Hkv", [(8, 16, 2), (1, 4, 4), (16, 16, 1), (3, 8, 2)])
def test_attn_matches_oracle(G, d, T, Hq, Hkv):
    B, Lmax = 3, 700
    ctx = [0, 65, Lmax - T]
    print_case(test="attn", B=B, T=T, Hq=Hq, Hkv=Hkv, d=d, Lmax=Lmax, ctx=ctx, seed=d + T)
    x = make_attn_inputs(B, T, Hq, Hkv, d, Lmax, ctx, seed=d + T, device=DEV)
    o, kc, vc = run(G, x)
    rel = check(x, o, kc, vc, 1.0 / d ** 0.5)
    print(f"  max error / max|v| = {rel:.2e}", flush=True)


@pytest.mark.parametrize("ctx", [1, 63, 64, 127, 128, 129, 511])
def test_attn_tile_edges(G, ctx):
    """Context lengths on and around the 64-key tile edges."""
    B, T, Hq, Hkv, d, Lmax = 1, 8, 16, 2, 256, 600
    print_case(test="attn_edges", ctx=ctx)
    x = make_attn_inputs(B, T, Hq, Hkv, d, Lmax, [ctx], seed=ctx, device=DEV)
    o, kc, vc = run(G, x)
    check(x, o, kc, vc, 1.0 / d ** 0.5)


def test_attn_sharp_scores(G):
    """A large scale makes the softmax nearly one-hot: the split merge and the
    running max must not lose the winning key."""
    B, T, Hq, Hkv, d, Lmax = 2, 8, 16, 2, 128, 2048
    print_case(test="attn_sharp", B=B, Lmax=Lmax)
    x = make_attn_inputs(B, T, Hq, Hkv, d, Lmax, [2000, 1500], seed=7, device=DEV)
    o, kc, vc = run(G, x, scale=1.0)
    check(x, o, kc, vc, 1.0)


def test_attn_out_of_range_ctx(G):
    """ctx outside [0, Lmax - T]: that instance gets NaN and no cache write; the
    others are computed."""
    B, T, Hq, Hkv, d, Lmax = 3, 8, 8, 2, 128, 300
    x = make_attn_inputs(B, T, Hq, Hkv, d, Lmax, [-1, 100, Lmax - T + 1], seed=9, device=DEV)
    o, kc, vc = run(G, x)
    assert torch.isnan(o[0]).all() and torch.isnan(o[2]).all()
    assert not torch.isnan(o[1]).any()
    assert torch.equal(kc[0], x.k_cache[0]) and torch.equal(kc[2], x.k_cache[2])


def test_attn_long_context_sampled_rows(G):
    """16 layers x (16 query / 2 key-value heads, d = 256), T = 8, 32,760 cached
    positions (the bench's shape): the outputs of sampled (layer, row, head)
    triples against the oracle computed for those triples alone."""
    B, T, Hq, Hkv, d, Lmax = 16, 8, 16, 2, 256, 32768
    ctx = Lmax - T
    print_case(test="attn_long", B=B, ctx=ctx)
    x = make_attn_inputs(B, T, Hq, Hkv, d, Lmax, [ctx] * B, seed=11, device=DEV, device_gen=True)
    o, kc, vc = run(G, x)
    rng = np.random.default_rng(3)
    scale = 1.0 / d ** 0.5
    vmax = float(x.v_cache.float().abs().max())
    for _ in range(12):
        b, t, h = int(rng.integers(B)), int(rng.integers(T)), int(rng.integers(Hq))
        g = h // (Hq // Hkv)
        keys = torch.cat([x.k_cache[b, :ctx, g], x.k_new[b, : t + 1, g]]).double().cpu().numpy()
        vals = torch.cat([x.v_cache[b, :ctx, g], x.v_new[b, : t + 1, g]]).double().cpu().numpy()
        s = keys @ x.q[b, t, h].double().cpu().numpy() * scale
        w = np.exp(s - s.max())
        ref = (w / w.sum()) @ vals
        err = np.abs(o[b, t, h].double().cpu().numpy() - ref).max()
        assert err <= TOL * vmax, (b, t, h, err)
    assert torch.equal(kc[:, ctx:ctx + T], x.k_new) and torch.equal(vc[:, ctx:ctx + T], x.v_new)
