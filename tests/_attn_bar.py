"""Per-output error bar for the full-attention verify kernel, derived from the
arithmetic the kernel performs.

What the kernel rounds.  q, k, v and the cache are bf16 and enter the products
exactly.  Each attention weight w_i = exp(s_i - m) (s_i = scale * q . k_i) is
formed in fp32; the running sum of the weights takes those fp32 values, while
the weighted sum of the values takes each weight rounded to bf16 (the MFMA
operand).  So, up to fp32 rounding,

    o_j = sum_i bf16(w_i) v_ij / sum_i w_i,
    o_j - ref_j = sum_i r_i w_i v_ij / sum_i w_i,

with r_i the relative rounding error of weight i: round-to-nearest-even to
8 significant bits gives |r_i| <= 2^-8.

The bar, per output element j of a row:

  * rounding of the weights to bf16.  The worst case, 2^-8 sum_i w_i |v_ij| /
    sum_i w_i, is about 2^-8 E|v|, larger than the outputs themselves once a
    row averages thousands of values: a bar built on it could not fail.  The
    errors r_i of distinct weights are independent, zero-mean and bounded, so
    Hoeffding's inequality bounds their sum: with c_i = 2^-8 w_i |v_ij| /
    sum w, P(|sum_i r_i w_i v_ij| / sum w >= t) <= 2 exp(-t^2 / (2 sum c_i^2)).
    t = sqrt(2 ln(2 / 1e-9)) * sqrt(sum c_i^2) = 6.55 sqrt(sum c_i^2) puts the
    chance that one element exceeds it at 1e-9.
  * fp32 work, worst case.  Each score is a d-term bf16 dot product
    accumulated in fp32, one rounding per 32 terms: |ds| <= (d/32 + 1) u
    scale sum_k |q_k k_ik|, u = 2^-24; its exponent in the log2 domain adds two
    roundings of |x| and exp2 one ulp.  Each weight is therefore off by at
    most eps_w (relative), in the numerator and the denominator alike.  The
    weighted sum rounds once per 32 keys and the running sum about once per
    64 keys and per lane reduction; the split merge a few times per split.
    These add (2 eps_w + (N/32 + N/64 + 64) u) sum_i w_i |v_ij| / sum_i w_i.

At 32,760 cached positions (d = 256, N(0, 1) keys and values) the bar is about
3e-4 against outputs of about 1e-2; leaving out one of the eight context
splits moves an output by about 2e-3, and halving one by half of it.
"""
import math

import numpy as np

U32 = 2.0 ** -24
BF16_REL = 2.0 ** -8
HOEFFDING = math.sqrt(2.0 * math.log(2.0 / 1e-9))


def attn_bar(q_row, keys, vals, scale):
    """q_row [d], keys/vals [N][d] (the positions the row sees) -> the bar on
    |o - ref| for each of the row's d outputs."""
    q = np.asarray(q_row, np.float64)
    K = np.asarray(keys, np.float64)
    V = np.asarray(vals, np.float64)
    N, d = K.shape
    s = K @ q * scale
    x = (s - s.max()) / math.log(2.0)                 # the kernel's log2-domain exponents
    w = np.exp(s - s.max())
    W = w.sum()
    absV = np.abs(V)
    mean_abs = (w @ absV) / W                         # sum_i w_i |v_ij| / sum w
    hoeff = HOEFFDING * BF16_REL * np.sqrt((w * w) @ (V * V)) / W
    dots = np.abs(K) @ np.abs(q)                      # sum_k |q_k k_ik| per key
    ds = (d / 32 + 1) * U32 * scale * dots.max()
    eps_w = math.log(2.0) * (ds / math.log(2.0) + 2 * U32 * np.abs(x).max()) + 2 * U32
    acc = (N / 32 + N / 64 + 64) * U32
    return hoeff + (2 * eps_w + acc) * mean_abs
