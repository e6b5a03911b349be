"""fp64 CPU oracle of the GDN mixer around the recurrence -- test
infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this module.  It shares no code with the HIP library.

Source: the README page ("How it works", region table, "GDN mixer" row): one
megakernel runs the layer's projections, recurrence, gating and normalisation
in dependency order; the audited-numbers page (DSpark section): a filter before
the mixer holds its last few inputs, which a rewind restores.  The pages give no formulas.  The
readings below follow the published Gated DeltaNet layer (Yang, Kautz &
Hatamizadeh, ICLR 2025), as deployed in the Qwen3-Next hybrid:

  * raw in-projection rows x_t [conv_dim], conv_dim = 2 Hk dk + H dv, channels
    [q heads | k heads | v heads]; a causal depthwise filter of width 4 over the
    history (the last 3 rows before the block, oldest first) and the block:
        y_t[c] = sum_{j=0..3} w[c][j] x_{t-3+j}[c],   then SiLU(y) = y sigmoid(y);
  * q, k, v are the channel groups; q and k are L2-normalised per head
    (u / sqrt(sum u^2 + 1e-6)); q is then scaled by 1/sqrt(dk);
  * value head h uses q/k head h / (H / Hk);
  * beta = sigmoid(b), g = -exp(A_log) softplus(a + dt_bias) (per head);
  * q, k, v are rounded to bf16 (round to nearest even) before the recurrence:
    the recurrence's operands are bf16;
  * after the recurrence, per token and head: y = o / sqrt(mean(o^2) + 1e-6) *
    norm_w * SiLU(z) (a gated RMS norm over the head's dv outputs).
"""
import numpy as np

EPS_L2 = 1e-6
EPS_RMS = 1e-6


def silu(x):
    x = np.asarray(x, np.float64)
    return x / (1.0 + np.exp(-x))


def softplus(x):
    x = np.asarray(x, np.float64)
    return np.log1p(np.exp(-np.abs(x))) + np.maximum(x, 0.0)


def bf16_round(x):
    """Round fp64 values to bf16 (round to nearest, ties to even), via fp32."""
    f = np.asarray(x, np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def prologue(x, hist, conv_w, a, b, A_log, dt_bias, Hk, dk, H, dv):
    """x [B][T][conv_dim], hist [B][3][conv_dim], conv_w [conv_dim][4], a, b [B][T][H],
    A_log, dt_bias [H] -> (q, k, v) fp64 [B][T][H][d] (per value head, already
    bf16-rounded) and (g, beta) [B][T][H]."""
    x = np.asarray(x, np.float64)
    hist = np.asarray(hist, np.float64)
    w = np.asarray(conv_w, np.float64)
    B, T, C = x.shape
    full = np.concatenate([hist, x], axis=1)            # rows: t - 3 .. T - 1
    y = np.zeros((B, T, C))
    for t in range(T):
        for j in range(4):
            y[:, t] += w[:, j] * full[:, t + j]
    y = silu(y)
    qh = y[..., : Hk * dk].reshape(B, T, Hk, dk)
    kh = y[..., Hk * dk: 2 * Hk * dk].reshape(B, T, Hk, dk)
    vh = y[..., 2 * Hk * dk:].reshape(B, T, H, dv)
    qh = qh / np.sqrt((qh ** 2).sum(-1, keepdims=True) + EPS_L2) / np.sqrt(dk)
    kh = kh / np.sqrt((kh ** 2).sum(-1, keepdims=True) + EPS_L2)
    grp = H // Hk
    q = bf16_round(np.repeat(qh, grp, axis=2))
    k = bf16_round(np.repeat(kh, grp, axis=2))
    v = bf16_round(vh)
    beta = 1.0 / (1.0 + np.exp(-np.asarray(b, np.float64)))
    g = -np.exp(np.asarray(A_log, np.float64)) * softplus(np.asarray(a, np.float64) + np.asarray(dt_bias, np.float64))
    return q, k, v, g, beta


def epilogue(o, z, norm_w):
    """o [B][T][H][dv], z [B][T][H][dv], norm_w [dv] -> gated RMS norm."""
    o = np.asarray(o, np.float64)
    rms = np.sqrt((o ** 2).mean(-1, keepdims=True) + EPS_RMS)
    return o / rms * np.asarray(norm_w, np.float64) * silu(z)
