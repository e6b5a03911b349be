"""fp64 CPU oracle of the verify pass's full-attention mixer -- test
infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares no code with the HIP library.

Source: the README page ("How it works", region table: the full-attention
mixer partitions the K/V context, accumulates online-softmax statistics locally
and merges the partial results before the output projection) and the
audited-numbers page ("How does lithos-metal fuse layer mixers on Metal?": 16 of
the 64 layers are full attention; workers keep small running softmax totals in
fp32 so the full score table is never written).  The oracle is the plain
definition those partial results must reproduce: softmax attention, computed
whole.

Readings:
  * The verify block's T rows are queries; each attends to the sequence's
    cached context (positions 0 .. ctx-1) and, causally, to the block's own rows
    0 .. t (their keys and values are the block's new rows).
  * Grouped queries: query head h reads key/value head h // (Hq / Hkv).
  * Scores are q . k * scale (scale given; 1/sqrt(d) in the workloads).
  * The block's new key/value rows are appended to the cache at positions
    ctx .. ctx+T-1; the cache's rewind is its length (the position the commit
    advances by n), so rows past the kept ones are simply overwritten later.
"""
import numpy as np


def attn_row(q_row, keys, vals, scale):
    """One query row: softmax over the visible keys of (keys . q_row * scale),
    then the weighted sum of their values.  q_row [d], keys/vals [N][d] (the
    visible positions, in order) -> [d]."""
    s = np.asarray(keys, np.float64) @ np.asarray(q_row, np.float64) * scale
    w = np.exp(s - s.max())
    return (w / w.sum()) @ np.asarray(vals, np.float64)


def attn_verify(q, k_new, v_new, k_cache, v_cache, ctx, scale):
    """q [B][T][Hq][d], k_new/v_new [B][T][Hkv][d], k_cache/v_cache
    [B][Lmax][Hkv][d], ctx [B] -> (o [B][T][Hq][d], k_cache', v_cache') with the
    block's rows written at ctx .. ctx+T-1."""
    q = np.asarray(q, np.float64)
    kn, vn = np.asarray(k_new, np.float64), np.asarray(v_new, np.float64)
    kc, vc = np.array(k_cache, np.float64), np.array(v_cache, np.float64)
    B, T, Hq, d = q.shape
    Hkv = kn.shape[2]
    group = Hq // Hkv
    o = np.zeros((B, T, Hq, d))
    for b in range(B):
        c = int(ctx[b])
        for t in range(T):
            for h in range(Hq):
                g = h // group
                keys = np.concatenate([kc[b, :c, g], kn[b, : t + 1, g]], axis=0)
                vals = np.concatenate([vc[b, :c, g], vn[b, : t + 1, g]], axis=0)
                o[b, t, h] = attn_row(q[b, t, h], keys, vals, scale)
        kc[b, c: c + T] = kn[b]
        vc[b, c: c + T] = vn[b]
    return o, kc, vc
