"""C-ABI checks that need no GPU: libgdn.so loads, exports every function that
include/gdn.h declares, and rejects bad host-side arguments with the documented
status before launching anything."""
import ctypes
import os
import re

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


@pytest.fixture(scope="module")
def G():
    so = os.path.join(ROOT, "speculative_verify_amd", "libgdn.so")
    if not os.path.exists(so):
        from speculative_verify_amd import build
        build.build()
    import speculative_verify_amd.gdn as G
    return G


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(G):
    names = declared_functions()
    assert len(names) >= 7
    assert sorted(G.EXPORTED) == names
    lib = ctypes.CDLL(G.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(G):
    for s in (0, -1, -2, -3, -4, -5, 17):
        assert len(G.strerror(s)) > 0


def _shape(B=1, H=2, dk=64, dv=64):
    import speculative_verify_amd.gdn as G
    return ctypes.byref(G.gdn_shape(B, H, dk, dv))


FAKE = ctypes.c_void_p(1 << 20)        # 16-byte aligned, never dereferenced
FAKE_ODD = ctypes.c_void_p((1 << 20) + 4)


def verify_call(G, S=FAKE, T=8, dt=0, shp=None, rec_bytes=1 << 30, q=FAKE, g=FAKE):
    return G.lib.gdn_verify_block(S, q, FAKE, FAKE, g, FAKE, T, dt, shp or _shape(), FAKE, FAKE,
                                  rec_bytes, None)


def test_verify_rejects_bad_arguments(G):
    assert verify_call(G, S=None) == -1
    assert verify_call(G, q=FAKE_ODD) == -1
    assert verify_call(G, dt=7) == -1
    assert verify_call(G, shp=_shape(dk=96)) == -2
    assert verify_call(G, shp=_shape(B=0)) == -2
    assert verify_call(G, shp=_shape(dv=32)) == -2
    assert verify_call(G, T=0) == -3
    assert verify_call(G, T=17) == -3
    need = G.lib.gdn_block_record_bytes(_shape(), 8, 0)
    assert verify_call(G, rec_bytes=need - 1) == -4
    assert G.lib.gdn_verify_block(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 0, None, FAKE, FAKE,
                                  1 << 30, None) == -1


def test_commit_and_prefill_reject_bad_arguments(G):
    assert G.lib.gdn_commit(None, FAKE, FAKE, None, _shape(), None) == -1
    assert G.lib.gdn_commit(FAKE, FAKE, None, None, _shape(), None) == -1
    assert G.lib.gdn_commit(FAKE, FAKE, FAKE, None, _shape(H=0), None) == -2
    pf = lambda L=64, chunk=64, dt=1, S=FAKE, shp=None: G.lib.gdn_prefill_chunked(
        S, FAKE, FAKE, FAKE, FAKE, FAKE, L, chunk, dt, shp or _shape(), FAKE, None, 0, None)
    assert pf(chunk=32) == -3
    assert pf(L=-1) == -3
    assert pf(dt=3) == -1
    assert pf(S=None) == -1
    assert pf(shp=_shape(dk=32)) == -2
    assert pf(L=0, S=None) == 0          # an empty prompt is a no-op
    assert G.lib.gdn_record_status(FAKE, _shape(), None, None) == -1


def test_commit_verify_rejects_bad_arguments(G):
    FAKE2 = ctypes.c_void_p(1 << 24)
    need = G.lib.gdn_block_record_bytes(_shape(), 8, 1)

    def cv(S=FAKE, rprev=FAKE2, rnext=FAKE, T=8, dt=1, shp=None, nbytes=1 << 20, n=FAKE):
        return G.lib.gdn_commit_verify(S, rprev, n, None, FAKE, FAKE, FAKE, FAKE, FAKE, T, dt,
                                       shp or _shape(), FAKE, rnext, nbytes, None)
    assert cv(S=None) == -1
    assert cv(n=None) == -1
    assert cv(rprev=FAKE) == -1                                  # the same record twice
    assert cv(rprev=ctypes.c_void_p((1 << 20) + 4096)) == -1      # record_prev inside record_next
    assert cv(rnext=ctypes.c_void_p((1 << 24) + 128)) == -1       # record_next over record_prev's header
    assert cv(dt=4) == -1
    assert cv(shp=_shape(dv=96)) == -2
    assert cv(T=0) == -3 and cv(T=17) == -3
    assert cv(nbytes=need - 1) == -4


def test_record_size_accounts_for_payload(G):
    for (B, H, dk, dv, T, dt) in [(1, 2, 64, 64, 8, torch.float32), (48, 32, 128, 128, 8, torch.bfloat16),
                                  (3, 5, 128, 64, 16, torch.bfloat16), (2, 1, 64, 128, 1, torch.float32)]:
        n = G.gdn_block_record_bytes(B, H, dk, dv, T, dt)
        es = 2 if dt == torch.bfloat16 else 4
        payload = B * T * H * (4 + 4 * dv + es * dk) + 16 * B + 16 * B * H
        assert payload < n <= payload + 6 * 256 + 256
        assert n % 256 == 0
    assert G.lib.gdn_block_record_bytes(_shape(), 0, 0) == 0
    assert G.lib.gdn_block_record_bytes(_shape(), 8, 5) == 0
    # Few heads: the two-pass schedule's workspace (Linv, P and gates per chunk).
    n = G.lib.gdn_prefill_workspace_bytes(_shape(B=1, H=32, dk=128, dv=128), 4096, 64)
    assert n >= 32 * 64 * (2 * 64 * 64 + 3 * 64) * 4 and n % 256 == 0
    # Many heads: one pass, no workspace.
    assert G.lib.gdn_prefill_workspace_bytes(_shape(B=48, H=32, dk=128, dv=128), 4096, 64) == 0
    assert G.lib.gdn_prefill_workspace_bytes(_shape(), 4096, 32) == 0


def _ashape(B=1, T=8, V=1000):
    import speculative_verify_amd.gdn as G
    return ctypes.byref(G.gdn_accept_shape(B, T, V))


def test_accept_and_rewind_reject_bad_arguments(G):
    L = G.lib
    big = 1 << 30
    ok = dict(tgt=FAKE, dt=1, drafts=FAKE, shp=None, n=FAKE, nxt=FAKE, ws=FAKE, wsb=big)

    def greedy(**kw):
        a = {**ok, **kw}
        return L.gdn_accept_greedy(a["tgt"], a["dt"], a["drafts"], a["shp"] or _ashape(), a["n"], a["nxt"],
                                   a["ws"], a["wsb"], None)

    assert greedy(tgt=None) == -1
    assert greedy(dt=7) == -1
    assert greedy(drafts=None) == -1
    assert greedy(ws=FAKE_ODD) == -1
    assert greedy(shp=_ashape(B=0)) == -2
    assert greedy(shp=_ashape(V=0)) == -2
    assert greedy(shp=_ashape(V=(1 << 26) + 1)) == -2
    assert greedy(shp=_ashape(T=0)) == -3
    assert greedy(shp=_ashape(T=17)) == -3
    assert greedy(wsb=16) == -4
    # T = 1: no drafts needed; still refused here for the workspace only.
    assert greedy(drafts=None, shp=_ashape(T=1), wsb=16) == -4

    def sampled(temp=1.0, wsb=big, draft=FAKE, shp=None):
        return L.gdn_accept_sampled(FAKE, draft, 1, FAKE, FAKE, FAKE, temp, shp or _ashape(), FAKE, FAKE, FAKE,
                                    wsb, None)

    assert sampled(temp=0.0) == -3
    assert sampled(temp=-1.0) == -3
    assert sampled(temp=float("inf")) == -3
    assert sampled(temp=float("nan")) == -3
    assert sampled(draft=None) == -1
    assert sampled(wsb=64) == -4
    assert L.gdn_accept_workspace_bytes(_ashape(), 1) > L.gdn_accept_workspace_bytes(_ashape(), 0) > 0
    assert L.gdn_accept_workspace_bytes(_ashape(T=0), 0) == 0

    # The call without a workspace: the same checks; a shape whose workspace
    # exceeds the library's per-device scratch is refused before any device work.
    def noalloc(temp=1.0, draft=FAKE, shp=None, n=FAKE):
        return L.gdn_accept_sampled_noalloc(FAKE, draft, 1, FAKE, FAKE, FAKE, temp, shp or _ashape(), n, FAKE,
                                            None)

    cap = L.gdn_accept_noalloc_max_bytes()
    assert cap == 1 << 20
    assert noalloc(temp=0.0) == -3 and noalloc(temp=float("nan")) == -3
    assert noalloc(draft=None) == -1 and noalloc(n=ctypes.c_void_p((1 << 20) + 2)) == -1
    assert noalloc(shp=_ashape(B=0)) == -2 and noalloc(shp=_ashape(T=17)) == -3
    fits = _ashape(B=96, T=8, V=151936)
    over = _ashape(B=128, T=8, V=151936)
    assert L.gdn_accept_workspace_bytes(fits, 1) <= cap < L.gdn_accept_workspace_bytes(over, 1)
    assert noalloc(shp=over) == -4

    def rewind(B=1, W=3, T=8, C=16, dt=1, hist=FAKE):
        return L.gdn_history_rewind(hist, FAKE, FAKE, B, W, T, C, dt, None)

    assert rewind(hist=None) == -1
    assert rewind(dt=5) == -1
    assert rewind(B=0) == -2
    assert rewind(C=0) == -2
    assert rewind(W=0) == -3
    assert rewind(W=17) == -3
    assert rewind(T=17) == -3


def test_attn_rejects_bad_arguments(G):
    L = G.lib

    def shp(B=1, Hq=16, Hkv=2, d=256, Lmax=1024):
        return ctypes.byref(G.gdn_attn_shape(B, Hq, Hkv, d, Lmax))

    def call(T=8, scale=0.0625, s=None, q=FAKE, ws=FAKE, wsb=1 << 40):
        return L.gdn_attn_verify(q, FAKE, FAKE, FAKE, FAKE, FAKE, T, scale, s or shp(), FAKE, ws, wsb, None)

    assert call(q=None) == -1
    assert call(ws=FAKE_ODD) == -1
    assert call(s=shp(d=64)) == -2
    assert call(s=shp(Hq=3, Hkv=2)) == -2
    assert call(s=shp(Hkv=0)) == -2
    assert call(s=shp(Lmax=4)) == -2
    assert call(s=shp(Hq=64, Hkv=2), T=16) == -2     # 16 x 32 query rows per key/value head
    assert call(T=0) == -3
    assert call(T=17) == -3
    assert call(scale=float("inf")) == -3
    assert call(wsb=16) == -4
    assert L.gdn_attn_workspace_bytes(shp(), 8) > 0
    assert L.gdn_attn_workspace_bytes(shp(d=64), 8) == 0


def test_mixer_rejects_bad_arguments(G):
    L = G.lib

    def mix(Hk=2, **kw):
        f = {n: FAKE for n in ("x", "history", "conv_w", "a", "b", "A_log", "dt_bias", "z", "norm_w")}
        f.update(kw)
        return ctypes.byref(G.gdn_mixer_inputs(*(f[n] for n in ("x", "history", "conv_w", "a", "b", "A_log",
                                                                 "dt_bias", "z", "norm_w")), Hk))

    def call(m=None, T=8, shp=None, S=FAKE, rec_bytes=1 << 30):
        return L.gdn_mixer_verify(S, m or mix(), T, shp or _shape(1, 4, 128, 128), FAKE, FAKE, rec_bytes, None)

    def fused(rp=FAKE, rn=ctypes.c_void_p(1 << 31), nb=1 << 20):
        return L.gdn_mixer_commit_verify(FAKE, rp, FAKE, None, mix(), 8, _shape(1, 4, 128, 128), FAKE, rn, nb, None)

    assert L.gdn_mixer_verify(FAKE, None, 8, _shape(1, 4, 128, 128), FAKE, FAKE, 1 << 30, None) == -1
    assert call(S=None) == -1
    assert call(m=mix(x=None)) == -1
    assert call(m=mix(x=FAKE_ODD)) == -1          # raw rows are copied in 16-byte pieces
    assert call(m=mix(history=FAKE_ODD)) == -1
    assert call(m=mix(norm_w=None)) == -1
    assert call(shp=_shape(1, 4, 64, 64)) == -2    # d = 128 only
    assert call(m=mix(Hk=3)) == -2                  # H not a multiple of Hk
    assert call(m=mix(Hk=0)) == -2
    assert call(T=0) == -3
    assert call(T=17) == -3
    assert call(rec_bytes=16) == -4
    assert fused(rn=FAKE) == -1                     # the two records overlap
    assert fused(nb=16) == -4
