"""Seeded synthetic inputs for the GDN verify / commit / prefill path.

This module holds only the data recipe (distributions, shapes, seeds).  It
contains none of the recurrence's arithmetic and is the one module that both
the HIP path's callers and the fp64 oracle's callers share.

The distributions stand in for the activations of a hybrid model's GDN layers
(48 GDN layers of 64, per the devdoido audit, "How does lithos-metal fuse
layer mixers on Metal?"; no dataset or weights are involved):

  q, k   N(0,1), L2-normalised per (token, head) in fp32, then rounded to the
         input dtype (bf16 round-to-nearest-even, or kept fp32)
  v      N(0,1), rounded to the input dtype
  beta   sigmoid(N(0,1)), fp32
  g      -softplus(N(0,1)) * g_scale, fp32 (log-decay; a = exp(g) in (0, 1])
  S0     0.02 * N(0,1), fp32 (0.02 is the standard deviation)
  n      Uniform{0..T}, int32 (accepted rows per verify block)

Draw order is fixed: S0, q, k, v, beta, g.  Inputs are drawn with a CPU
torch.Generator (bit-reproducible everywhere) unless ``device_gen`` is set,
in which case large tensors are drawn on the device and the oracle receives
copies of the exact bytes.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch


@dataclass
class GdnInputs:
    S0: torch.Tensor     # fp32 [B][H][dv][dk]
    q: torch.Tensor      # [B][L][H][dk]
    k: torch.Tensor      # [B][L][H][dk]
    v: torch.Tensor      # [B][L][H][dv]
    g: torch.Tensor      # fp32 [B][L][H]
    beta: torch.Tensor   # fp32 [B][L][H]

    def to(self, device) -> "GdnInputs":
        return GdnInputs(*(getattr(self, f).to(device) for f in ("S0", "q", "k", "v", "g", "beta")))

    @property
    def shape(self):
        B, H, dv, dk = self.S0.shape
        return B, H, dk, dv, self.q.shape[1]


def _normalise(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def make_inputs(B: int, H: int, dk: int, dv: int, L: int, *, dtype=torch.bfloat16,
                seed: int = 0, device="cpu", g_scale: float = 1.0,
                s0_std: float = 0.02, device_gen: bool = False) -> GdnInputs:
    """Draw one set of inputs with the recipe above."""
    gen_dev = torch.device(device) if device_gen else torch.device("cpu")
    gen = torch.Generator(device=gen_dev)
    gen.manual_seed(int(seed))

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=gen_dev, dtype=torch.float32)

    S0 = s0_std * randn(B, H, dv, dk)
    q = _normalise(randn(B, L, H, dk)).to(dtype)
    k = _normalise(randn(B, L, H, dk)).to(dtype)
    v = randn(B, L, H, dv).to(dtype)
    beta = torch.sigmoid(randn(B, L, H))
    g = -torch.nn.functional.softplus(randn(B, L, H)) * g_scale
    out = GdnInputs(S0, q, k, v, g.contiguous(), beta.contiguous())
    return out.to(device) if gen_dev != torch.device(device) else out


def make_accepts(count: int, T: int, *, seed: int = 0) -> torch.Tensor:
    """Accepted-row counts n ~ Uniform{0..T}, int32, drawn on the CPU."""
    gen = torch.Generator()
    gen.manual_seed(int(seed) + 7919)
    return torch.randint(0, T + 1, (count,), generator=gen, dtype=torch.int32)


def make_accepts_paired(count: int, T: int, *, seed: int = 0) -> torch.Tensor:
    """Accepted-row counts in pairs (n, T - n) with n ~ Uniform{0..T}: each entry is
    still Uniform{0..T}, and every window that starts at an even index and has an
    even length averages exactly T / 2, so a timed window's token count does not
    depend on the luck of the draw.  An odd count ends with T // 2."""
    half = make_accepts((count + 1) // 2, T, seed=seed)
    out = torch.stack([half, T - half], dim=1).flatten()[:count].clone()
    if count % 2:
        out[-1] = T // 2
    return out.to(torch.int32)


# ---------------------------------------------------------------------------
# Acceptance inputs: logits of one verify block per sequence, standing in for a
# target model and its drafter (no weights or vocabulary file involved).
#
#   target logits  N(0,1) per entry, plus `peak` on `n_peak` random entries per
#                  row (a few likely tokens over a flat tail, the shape of a
#                  language model's next-token distribution)
#   drafter logits the target's rows 0 .. T-2 plus drift * N(0,1) (a drafter
#                  close to its target)
#   draft tokens   drawn from softmax(drafter / tau) by the Gumbel-max rule:
#                  argmax(drafter / tau - log(-log U)), U uniform
#   u_accept, u_sample   U[0, 1)
# With ``plan_greedy`` each sequence instead draws k ~ Uniform{0..T-1}; row j
# gets a planted top entry (one random entry raised to 1 above the row's
# maximum), drafts j < k copy it and draft k (when k < T - 1) is another entry.
# Logits are rounded to ``dtype`` last.  Draw order: target, peaks, drafter,
# Gumbel noise, u_accept, u_sample (or target, plan).
# ---------------------------------------------------------------------------
@dataclass
class AcceptInputs:
    target: torch.Tensor     # [B][T][V]
    draft: torch.Tensor      # [B][T-1][V]
    tokens: torch.Tensor     # int32 [B][T-1]
    u_accept: torch.Tensor   # fp32 [B][T-1]
    u_sample: torch.Tensor   # fp32 [B]

    def to(self, device) -> "AcceptInputs":
        return AcceptInputs(*(getattr(self, f).to(device)
                              for f in ("target", "draft", "tokens", "u_accept", "u_sample")))


def make_accept_inputs(B: int, T: int, V: int, *, dtype=torch.bfloat16, seed: int = 0, device="cpu",
                       tau: float = 1.0, peak: float = 8.0, n_peak: int = 4, drift: float = 0.5,
                       plan_greedy: bool = False) -> AcceptInputs:
    gen = torch.Generator()
    gen.manual_seed(int(seed) + 104729)
    f32 = torch.float32
    target = torch.randn(B, T, V, generator=gen, dtype=f32)
    if plan_greedy:
        k = torch.randint(0, T, (B,), generator=gen)
        top = torch.randint(0, V, (B, T), generator=gen)
        other = torch.randint(0, max(V - 1, 1), (B, T), generator=gen)
        rmax = target.max(dim=2).values
        target.scatter_(2, top.unsqueeze(2), (rmax + 1.0).unsqueeze(2))
        tokens = torch.empty(B, max(T - 1, 0), dtype=torch.int32)
        for b in range(B):
            for j in range(T - 1):
                if j < int(k[b]):
                    tokens[b, j] = top[b, j]
                else:   # any entry but the planted one
                    o = int(other[b, j])
                    tokens[b, j] = o + 1 if o >= int(top[b, j]) and V > 1 else o
        draft = target[:, : T - 1].clone()
        u_acc = torch.zeros(B, max(T - 1, 0), dtype=f32)
        u_smp = torch.zeros(B, dtype=f32)
    else:
        if n_peak > 0 and peak != 0.0:
            idx = torch.randint(0, V, (B, T, n_peak), generator=gen)
            target.scatter_add_(2, idx, torch.full((B, T, n_peak), float(peak)))
        draft = target[:, : T - 1] + drift * torch.randn(B, max(T - 1, 0), V, generator=gen, dtype=f32)
        draft = draft.to(dtype).to(f32)
        gum = -torch.log(-torch.log(torch.rand(B, max(T - 1, 0), V, generator=gen, dtype=f32).clamp_min(1e-30)))
        tokens = torch.argmax(draft / tau + gum, dim=2).to(torch.int32)
        u_acc = torch.rand(B, max(T - 1, 0), generator=gen, dtype=f32)
        u_smp = torch.rand(B, generator=gen, dtype=f32)
    out = AcceptInputs(target.to(dtype).contiguous(), draft.to(dtype).contiguous(), tokens.contiguous(),
                       u_acc.contiguous(), u_smp.contiguous())
    return out.to(device)


def make_history_inputs(B: int, W: int, T: int, C: int, *, dtype=torch.bfloat16, seed: int = 0, device="cpu"):
    """Filter history [B][W][C] and the block's filter inputs [B][T][C], N(0,1)."""
    gen = torch.Generator()
    gen.manual_seed(int(seed) + 1299709)
    hist = torch.randn(B, W, C, generator=gen).to(dtype)
    rows = torch.randn(B, T, C, generator=gen).to(dtype)
    return hist.to(device), rows.to(device)


# ---------------------------------------------------------------------------
# Full-attention inputs: one verify block's queries, its new keys and values,
# and a key/value cache, all N(0,1) rounded to bf16 (cache rows past ctx hold
# N(0,1) too: they must not be read).  Draw order: q, k_new, v_new, k_cache,
# v_cache.  Drawn on the CPU generator, or on the device with device_gen.
# ---------------------------------------------------------------------------
@dataclass
class AttnInputs:
    q: torch.Tensor        # bf16 [B][T][Hq][d]
    k_new: torch.Tensor    # bf16 [B][T][Hkv][d]
    v_new: torch.Tensor
    k_cache: torch.Tensor  # bf16 [B][Lmax][Hkv][d]
    v_cache: torch.Tensor
    ctx: torch.Tensor      # int32 [B]

    def to(self, device) -> "AttnInputs":
        return AttnInputs(*(getattr(self, f).to(device) for f in ("q", "k_new", "v_new", "k_cache", "v_cache", "ctx")))


def make_attn_inputs(B: int, T: int, Hq: int, Hkv: int, d: int, Lmax: int, ctx, *, seed: int = 0, device="cpu",
                     device_gen: bool = False) -> AttnInputs:
    gen_dev = torch.device(device) if device_gen else torch.device("cpu")
    gen = torch.Generator(device=gen_dev)
    gen.manual_seed(int(seed) + 15485863)

    def randn(*shape):
        return torch.randn(*shape, generator=gen, device=gen_dev, dtype=torch.float32).to(torch.bfloat16)

    out = AttnInputs(randn(B, T, Hq, d), randn(B, T, Hkv, d), randn(B, T, Hkv, d), randn(B, Lmax, Hkv, d),
                     randn(B, Lmax, Hkv, d), torch.as_tensor(ctx, dtype=torch.int32).reshape(B).to(gen_dev))
    return out.to(device) if gen_dev != torch.device(device) else out


# ---------------------------------------------------------------------------
# GDN mixer inputs (the layer's raw in-projection rows and the mixer's
# parameters; random, no trained weights): x and the filter history N(0,1) in
# bf16; filter taps 0.5 N(0,1); the gate pre-activations a, b N(0,1); A_log and
# dt_bias 0.5 N(0,1); the output gate z N(0,1) in bf16; the norm weight
# 1 + 0.1 N(0,1).  conv_dim = 2 Hk d + H d.  Draw order as listed.
# ---------------------------------------------------------------------------
@dataclass
class MixerInputs:
    x: torch.Tensor        # bf16 [B][T][conv_dim]
    history: torch.Tensor  # bf16 [B][3][conv_dim]
    conv_w: torch.Tensor   # fp32 [conv_dim][4]
    a: torch.Tensor        # fp32 [B][T][H]
    b: torch.Tensor        # fp32 [B][T][H]
    A_log: torch.Tensor    # fp32 [H]
    dt_bias: torch.Tensor  # fp32 [H]
    z: torch.Tensor        # bf16 [B][T][H][d]
    norm_w: torch.Tensor   # fp32 [d]
    Hk: int

    def to(self, device) -> "MixerInputs":
        f = ("x", "history", "conv_w", "a", "b", "A_log", "dt_bias", "z", "norm_w")
        return MixerInputs(*(getattr(self, n).to(device) for n in f), self.Hk)

    def block(self, r: int, T: int) -> "MixerInputs":
        """Rows r T .. r T + T - 1 of a longer draw (the history left as drawn)."""
        sl = lambda t: t[:, r * T:(r + 1) * T].contiguous()
        return MixerInputs(sl(self.x), self.history, self.conv_w, sl(self.a), sl(self.b), self.A_log,
                           self.dt_bias, sl(self.z), self.norm_w, self.Hk)


def make_mixer_inputs(B: int, T: int, H: int, Hk: int, d: int = 128, *, seed: int = 0, device="cpu") -> MixerInputs:
    gen = torch.Generator()
    gen.manual_seed(int(seed) + 32452843)
    cdim = 2 * Hk * d + H * d
    rn = lambda *s: torch.randn(*s, generator=gen, dtype=torch.float32)
    out = MixerInputs(rn(B, T, cdim).to(torch.bfloat16), rn(B, 3, cdim).to(torch.bfloat16), 0.5 * rn(cdim, 4),
                      rn(B, T, H), rn(B, T, H), 0.5 * rn(H), 0.5 * rn(H), rn(B, T, H, d).to(torch.bfloat16),
                      1.0 + 0.1 * rn(d), Hk)
    return out.to(device)
