"""fp64 CPU oracle of on-device acceptance and rewind -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares no code with the HIP library.

Source: the audited-numbers page ("Qwen 3.8 27B mac m5: 200 tok/s, audited"),
section "How does DSpark speculative decoding create more than one token per
read?": acceptance is exact speculative sampling.  In greedy mode a drafted
token is kept only where it equals the target model's token; in sampled mode it
is kept with probability min(1, p/q) (target probability over drafter
probability); the pass then emits a correction token at the first rejection, or
a bonus token when every draft was kept.  Rewind follows: the key-value cache,
the last few inputs held by the filter before the mixer, and the recurrent state
all return to the kept tokens.  The README page ("How it works") keeps
positions, accepted tokens and commit/rollback on the GPU.

Readings (where the pages leave a step open):
  * The verify block's rows are [anchor, d_1, ..., d_{T-1}]: the last confirmed
    token and T - 1 drafted tokens.  Target row t's logits give the distribution
    of the token after row t; drafter row j (0 .. T-2) is the distribution d_{j+1}
    was drawn from.
  * p = softmax(target logits / tau), q = softmax(drafter logits / tau), one
    temperature tau > 0 for both.
  * Draft j + 1 is kept iff u_j * q(d) < p(d) (u_j uniform in [0, 1): the same
    event as u_j < min(1, p/q), written without the division).
  * The correction token is drawn from max(0, p - q) normalised, at the row of the
    first rejection; the bonus token from p of the last target row.
  * A draw from weights w with uniform u is the smallest index x with
    w_0 + ... + w_x > u * (w_0 + ... + w_{V-1}).
  * Rows committed to the recurrent state: n = 1 + m (the anchor and the m kept
    drafts); the emitted correction or bonus token is the next pass's anchor.
  * Greedy ties take the lowest index.
  * The filter layer's history is the last W rows of its input; after the pass it
    is the last W rows of [old history; block rows 0 .. n-1].
All random numbers are inputs (u_accept [B][T-1], u_sample [B]).
"""
import numpy as np


def softmax(z, tau):
    """softmax(z / tau) in fp64."""
    x = np.asarray(z, dtype=np.float64) / float(tau)
    e = np.exp(x - x.max())
    return e / e.sum()


def first_argmax(z):
    """Index of the largest value, the lowest index among equals."""
    z = np.asarray(z, dtype=np.float64)
    return int(np.flatnonzero(z == z.max())[0])


def draw(w, u):
    """Smallest x with cumsum(w)[x] > u * sum(w); also the distance of u * sum(w)
    to the nearest cumulative boundary, relative to sum(w) (how close the draw is
    to a tie)."""
    w = np.asarray(w, dtype=np.float64)
    c = np.cumsum(w)
    t = float(u) * c[-1]
    x = int(np.searchsorted(c, t, side="right"))
    x = min(x, len(w) - 1)
    lo = c[x - 1] if x > 0 else 0.0
    margin = min(abs(t - lo), abs(c[x] - t)) / c[-1]
    return x, margin


def accept_greedy(target_logits, draft_tokens):
    """target_logits [B][T][V], draft_tokens [B][T-1] -> (n [B], next_token [B])."""
    z = np.asarray(target_logits, dtype=np.float64)
    d = np.asarray(draft_tokens)
    B, T, _ = z.shape
    n = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    for b in range(B):
        m = 0
        while m < T - 1 and int(d[b, m]) == first_argmax(z[b, m]):
            m += 1
        n[b] = m + 1
        nxt[b] = first_argmax(z[b, m])
    return n, nxt


def accept_sampled(target_logits, draft_logits, draft_tokens, u_accept, u_sample, tau, flip=None):
    """Exact speculative sampling over one verify block per sequence.

    target_logits [B][T][V], draft_logits [B][T-1][V], draft_tokens [B][T-1],
    u_accept [B][T-1], u_sample [B]  ->  (n [B], next_token [B], info), where
    info[b] = dict(m=kept drafts, kind="correction"|"bonus", accept_margins=[...],
    draw_margin=...).  An accept margin is |u q(d) - p(d)| / max(p(d), q(d)): how
    far that decision is from its threshold.

    flip: optional {b: set of draft indices}; those keep decisions of sequence b
    go the other way.  A decision within rounding of its threshold can go either
    way in a lower precision, and this gives the outcome on the other branch."""
    z = np.asarray(target_logits, dtype=np.float64)
    y = np.asarray(draft_logits, dtype=np.float64)
    d = np.asarray(draft_tokens)
    ua = np.asarray(u_accept, dtype=np.float64)
    us = np.asarray(u_sample, dtype=np.float64)
    B, T, _ = z.shape
    n = np.zeros(B, np.int32)
    nxt = np.zeros(B, np.int32)
    info = []
    for b in range(B):
        m, margins = 0, []
        p = q = None
        while m < T - 1:
            p = softmax(z[b, m], tau)
            q = softmax(y[b, m], tau)
            tok = int(d[b, m])
            lhs, rhs = ua[b, m] * q[tok], p[tok]
            margins.append(abs(lhs - rhs) / max(p[tok], q[tok], 1e-300))
            keep = lhs < rhs
            if flip is not None and m in flip.get(b, ()):
                keep = not keep
            if keep:
                m += 1
            else:
                break
        if m < T - 1:
            w, kind = np.maximum(p - q, 0.0), "correction"
        else:
            w, kind = softmax(z[b, T - 1], tau), "bonus"
        x, dm = draw(w, us[b])
        n[b] = m + 1
        nxt[b] = x
        info.append(dict(m=m, kind=kind, accept_margins=margins, draw_margin=dm))
    return n, nxt, info


def conv_window_rewind(window, rows, n):
    """window [B][W][C] (history before the block), rows [B][T][C] (the block's
    filter inputs), n [B] in [0, T] -> the history after keeping n rows: the last
    W rows of [window[b]; rows[b, :n[b]]]."""
    win = np.asarray(window)
    blk = np.asarray(rows)
    B, W, _ = win.shape
    out = np.empty_like(win)
    for b in range(B):
        seq = np.concatenate([win[b], blk[b, : int(n[b])]], axis=0)
        out[b] = seq[seq.shape[0] - W:]
    return out
