"""gdn_accept_sampled_noalloc (the library's own per-device scratch, nothing
allocated at call time) against gdn_accept_sampled with a caller's workspace,
through libgdn's C ABI: two calls in a row, the second smaller than the first
(the scratch keeps the first call's contents), each bit-exact against the
workspace call on the same inputs (n and the emitted token are integers, so
the bar is equality), and against the oracle's outcome where its decisions are
clear of fp32 rounding."""
import numpy as np
import pytest
import torch

from oracle import accept_oracle as A
from speculative_verify_amd.inputs import make_accept_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def G():
    import speculative_verify_amd.gdn as G
    assert torch.cuda.is_available(), "the gpu tests need a GPU"
    return G


def run(G, x, tau, noalloc):
    B = x.target.shape[0]
    n = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    nxt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    call = G.gdn_accept_sampled_noalloc if noalloc else G.gdn_accept_sampled
    call(x.target, x.draft, x.tokens, x.u_accept, x.u_sample, tau, n, nxt)
    torch.cuda.synchronize()
    return n.cpu().numpy(), nxt.cpu().numpy()


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
def test_noalloc_matches_the_workspace_call(G, dtype):
    for B, T, V, tau, seed in ((64, 8, 151936, 1.0, 31), (3, 4, 5000, 0.8, 32)):
        print(f"case: test=noalloc B={B} T={T} V={V} tau={tau} dtype={dtype} seed={seed}", flush=True)
        x = make_accept_inputs(B, T, V, dtype=dtype, seed=seed, device=DEV, tau=tau, peak=12.0)
        n_na, x_na = run(G, x, tau, True)
        n_ws, x_ws = run(G, x, tau, False)
        assert np.array_equal(n_na, n_ws) and np.array_equal(x_na, x_ws)
        xc = x.to("cpu")
        rn, rx, info = A.accept_sampled(xc.target.float().numpy(), xc.draft.float().numpy(), xc.tokens.numpy(),
                                        xc.u_accept.numpy(), xc.u_sample.numpy(), tau)
        clear = [b for b in range(B) if min(info[b]["accept_margins"], default=1.0) >= 1e-4
                 and info[b]["draw_margin"] >= 2e-5]
        assert len(clear) >= B // 2
        assert all(n_na[b] == rn[b] and x_na[b] == rx[b] for b in clear)


def test_noalloc_refuses_a_shape_beyond_its_scratch(G):
    B, T, V = 128, 8, 151936
    x = make_accept_inputs(2, T, 1000, dtype=torch.bfloat16, seed=3, device=DEV)
    big = torch.empty(B, T, V, dtype=torch.bfloat16, device=DEV)
    n = torch.empty(B, dtype=torch.int32, device=DEV)
    with pytest.raises(G.GdnError):
        G.gdn_accept_sampled_noalloc(big, big[:, : T - 1].contiguous(), torch.zeros(B, T - 1, dtype=torch.int32,
                                     device=DEV), torch.zeros(B, T - 1, device=DEV), torch.zeros(B, device=DEV),
                                     1.0, n, n.clone())
    del x
