"""GPU parity of the verify pass's full-attention mixer (gdn_attn_verify)
against the fp64 oracle (oracle/attn_oracle.py), through libgdn's C ABI.

Bar: |o - ref| <= attn_bar(row) for every output element, the per-row bound
that tests/_attn_bar.py derives from the kernel's arithmetic (the weights
rounded to bf16 in the P V product, fp32 everywhere else).  At the benchmark's
32,760 cached positions it is about 3e-4 against outputs of about 1e-2, and
tests/test_attn_bar.py shows on the CPU that an output with one context split
left out fails it.  The cache append is bit-exact.
"""
import numpy as np
import pytest
import torch

from oracle import attn_oracle as A
from speculative_verify_amd.inputs import make_attn_inputs
from tests._attn_bar import attn_bar

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


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


def check_row(o_row, q_row, keys, vals, scale, where):
    """One query row against the oracle, within the derived bar; returns the
    worst error over the bar."""
    ref = A.attn_row(q_row, keys, vals, scale)
    bar = attn_bar(q_row, keys, vals, scale)
    err = np.abs(np.asarray(o_row, np.float64) - ref)
    assert (err <= bar).all(), (where, float((err / bar).max()), float(err.max()), float(np.abs(ref).max()))
    return float((err / bar).max())


def check(x, o, kc, vc, scale):
    """Every output row within its bar; the block's rows in the cache, every other
    cache row untouched."""
    xc = x.to("cpu")
    f = lambda t: t.double().numpy()
    q, kn, vn, kcache, vcache = f(xc.q), f(xc.k_new), f(xc.v_new), f(xc.k_cache), f(xc.v_cache)
    oc = o.cpu().double().numpy()
    B, T, Hq, _ = q.shape
    group = Hq // kn.shape[2]
    worst = 0.0
    for b in range(B):
        c = int(xc.ctx[b])
        for t in range(T):
            for h in range(Hq):
                g = h // group
                keys = np.concatenate([kcache[b, :c, g], kn[b, : t + 1, g]])
                vals = np.concatenate([vcache[b, :c, g], vn[b, : t + 1, g]])
                worst = max(worst, check_row(oc[b, t, h], q[b, t, h], keys, vals, scale, (b, t, h)))
    _, rk, rv = A.attn_verify(q, kn, vn, kcache, vcache, xc.ctx.numpy(), scale)
    assert np.array_equal(kc.cpu().float().numpy(), rk)
    assert np.array_equal(vc.cpu().float().numpy(), rv)
    return worst


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("T,Hq,Hkv", [(8, 16, 2), (1, 4, 4), (16, 16, 1), (3, 8, 2)])
def test_attn_matches_oracle(G, d, T, Hq, Hkv):
    B, Lmax = 3, 700
    ctx = [0, 65, Lmax - T]
    print_case(test="attn", B=B, T=T, Hq=Hq, Hkv=Hkv, d=d, Lmax=Lmax, ctx=ctx, seed=d + T)
    x = make_attn_inputs(B, T, Hq, Hkv, d, Lmax, ctx, seed=d + T, device=DEV)
    o, kc, vc = run(G, x)
    worst = check(x, o, kc, vc, 1.0 / d ** 0.5)
    print(f"  max error / bar = {worst:.3f}", flush=True)


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
    positions (the benchmark's shape and launch): 48 sampled (layer, row, head)
    outputs against the oracle's rows, each within its derived bar."""
    B, T, Hq, Hkv, d, Lmax = 16, 8, 16, 2, 256, 32768
    ctx = Lmax - T
    print_case(test="attn_long", B=B, ctx=ctx, rows=48)
    x = make_attn_inputs(B, T, Hq, Hkv, d, Lmax, [ctx] * B, seed=11, device=DEV, device_gen=True)
    o, kc, vc = run(G, x)
    rng = np.random.default_rng(3)
    scale = 1.0 / d ** 0.5
    G_ = Hq // Hkv
    oc = o.cpu().double().numpy()
    worst = 0.0
    # Six (layer, key/value head) slabs, eight rows each: every block row t once,
    # a random query head of the group.
    for b, g in zip(rng.choice(B, 6, replace=False), rng.integers(0, Hkv, 6)):
        b, g = int(b), int(g)
        kcache = x.k_cache[b, :ctx, g].double().cpu().numpy()
        vcache = x.v_cache[b, :ctx, g].double().cpu().numpy()
        kn, vn = x.k_new[b, :, g].double().cpu().numpy(), x.v_new[b, :, g].double().cpu().numpy()
        for t in range(T):
            h = g * G_ + int(rng.integers(G_))
            keys, vals = np.concatenate([kcache, kn[: t + 1]]), np.concatenate([vcache, vn[: t + 1]])
            worst = max(worst, check_row(oc[b, t, h], x.q[b, t, h].double().cpu().numpy(), keys, vals, scale,
                                         (b, t, h)))
    print(f"  max error / bar = {worst:.3f}", flush=True)
    assert torch.equal(kc[:, ctx:ctx + T], x.k_new) and torch.equal(vc[:, ctx:ctx + T], x.v_new)
