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
