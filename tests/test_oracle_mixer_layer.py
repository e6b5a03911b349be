"""The mixer oracle's readings against the published layer they follow.

The pages give no formulas for the GDN mixer; the oracle (oracle/mixer_oracle.py
with the recurrence of oracle/gdn_oracle.c) reads them from the Gated DeltaNet
layer as the Qwen3-Next hybrid deploys it.  transformers ships that layer
(Qwen3NextGatedDeltaNet) with plain-PyTorch references of its pieces (l2norm,
Qwen3NextRMSNormGated, torch_recurrent_gated_delta_rule), so each reading is
checked here against the layer itself, on small random inputs, CPU only:

  * the filter, SiLU, L2 norms, the 1/sqrt(dk) query scale and the grouped
    heads (readings of the raw rows' layout, the width-4 causal filter with its
    history, q/k normalisation and head grouping): the layer's own q, k, v,
    captured where it hands them to the recurrence, agree with the oracle's
    prologue to 1e-12 in fp64 (the oracle's bf16 rounding of its operands
    switched off for the comparison, and on again: its bf16 values are the
    layer's values rounded);
  * beta = sigmoid(b) to 1e-12; g = -exp(A_log) softplus(a + dt_bias) to fp32
    precision (the layer casts the gate parameters to fp32);
  * the recurrence: the oracle's sequential fp64 definition against
    torch_recurrent_gated_delta_rule, with the state transposed (the layer keeps
    it as [dk][dv]) and the query scale mapped (the layer scales q inside, the
    plain calls take q as given); the reference computes in fp32, so the bar is
    fp32's;
  * the gated RMS norm against Qwen3NextRMSNormGated (fp32 inside);
  * end to end: the layer's forward (projection rows in, gated norm out; the
    output projection replaced by the identity) against prologue, recurrence
    and epilogue over the same rows from a zero state and a zero history.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import mixer_oracle as M

tq = pytest.importorskip("transformers.models.qwen3_next.modeling_qwen3_next")
from transformers import Qwen3NextConfig  # noqa: E402

HK, H, DK, DV, HID = 2, 4, 16, 16, 64
FP32_BAR = 2e-5


def _layer(seed):
    torch.manual_seed(seed)
    cfg = Qwen3NextConfig(hidden_size=HID, linear_num_key_heads=HK, linear_num_value_heads=H,
                          linear_key_head_dim=DK, linear_value_head_dim=DV, linear_conv_kernel_dim=4,
                          num_hidden_layers=1, rms_norm_eps=1e-6)
    layer = tq.Qwen3NextGatedDeltaNet(cfg, layer_idx=0).double()
    with torch.no_grad():
        layer.conv1d.weight.normal_(0.0, 0.5)
        layer.A_log.normal_(0.0, 0.5)
        layer.dt_bias.normal_(0.0, 0.5)
        layer.norm.weight.copy_(1.0 + 0.1 * torch.randn(DV, dtype=torch.float64))
        layer.in_proj_qkvz.weight.normal_(0.0, 0.3)
        layer.in_proj_ba.weight.normal_(0.0, 0.5)
    layer.out_proj = torch.nn.Identity()
    return layer


def _raw(layer, h):
    """The layer's in-projection rows in the oracle's layout ([q heads | k heads |
    v heads] per token), and z, a, b, from the layer's own projections."""
    with torch.no_grad():
        q, k, v, z, b, a = layer.fix_query_key_value_ordering(layer.in_proj_qkvz(h), layer.in_proj_ba(h))
        B, L = h.shape[:2]
        x = torch.cat([q.reshape(B, L, -1), k.reshape(B, L, -1), v.reshape(B, L, -1)], dim=-1)
    return x.numpy(), z.numpy(), a.numpy(), b.numpy()


def _capture(monkeypatch):
    """Record what the layer hands to its recurrence; run the recurrent reference
    in its place."""
    seen = {}

    def chunk_rule(query, key, value, g, beta, initial_state, output_final_state, use_qk_l2norm_in_kernel, **kw):
        seen.update(q=query.detach().clone(), k=key.detach().clone(), v=value.detach().clone(),
                    g=g.detach().clone(), beta=beta.detach().clone(), l2=use_qk_l2norm_in_kernel)
        o, s = tq.torch_recurrent_gated_delta_rule(query, key, value, g=g, beta=beta, initial_state=initial_state,
                                                   output_final_state=output_final_state,
                                                   use_qk_l2norm_in_kernel=use_qk_l2norm_in_kernel)
        return o.to(value.dtype), s

    monkeypatch.setattr(tq, "torch_chunk_gated_delta_rule", chunk_rule)
    return seen


def _rel(x, r):
    x, r = np.asarray(x, np.float64), np.asarray(r, np.float64)
    return float(np.abs(x - r).max() / np.abs(r).max())


def test_prologue_matches_the_layer(monkeypatch):
    layer = _layer(1)
    B, T = 2, 9
    h = torch.randn(B, 3 + T, HID, dtype=torch.float64)
    seen = _capture(monkeypatch)
    with torch.no_grad():
        layer(h)
    assert seen["l2"]            # q and k are L2-normalised inside the recurrence call
    x, z, a, b = _raw(layer, h)
    # The layer filters the whole sequence from a zero history; the oracle takes
    # rows 0 .. 2 as the block's history.
    args = (x[:, 3:], x[:, :3], layer.conv1d.weight[:, 0, :].detach().numpy(), a[:, 3:], b[:, 3:],
            layer.A_log.detach().numpy(), layer.dt_bias.detach().numpy(), HK, DK, H, DV)
    ref_q = tq.l2norm(seen["q"], dim=-1, eps=1e-6).numpy()[:, 3:] / math.sqrt(DK)
    ref_k = tq.l2norm(seen["k"], dim=-1, eps=1e-6).numpy()[:, 3:]
    ref_v = seen["v"].numpy()[:, 3:]
    with monkeypatch.context() as mp:
        mp.setattr(M, "bf16_round", lambda u: np.asarray(u, np.float64))
        q, k, v, g, beta = M.prologue(*args)
    assert _rel(q, ref_q) <= 1e-12 and _rel(k, ref_k) <= 1e-12 and _rel(v, ref_v) <= 1e-12
    assert _rel(beta, seen["beta"].numpy()[:, 3:]) <= 1e-12
    assert _rel(g, seen["g"].numpy()[:, 3:]) <= 1e-6
    q16, k16, v16, _, _ = M.prologue(*args)
    assert np.array_equal(q16, M.bf16_round(ref_q)) and np.array_equal(k16, M.bf16_round(ref_k))
    assert np.array_equal(v16, M.bf16_round(ref_v))


def test_recurrence_matches_the_layers_reference():
    rng = np.random.default_rng(2)
    B, T = 2, 12
    q = rng.normal(size=(B, T, H, DK))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.normal(size=(B, T, H, DK))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(B, T, H, DV))
    g = -np.log1p(np.exp(rng.normal(size=(B, T, H))))
    beta = 1 / (1 + np.exp(-rng.normal(size=(B, T, H))))
    S0 = 0.3 * rng.normal(size=(B, H, DV, DK))
    o, S = oracle.prefill_seq(S0, q, k, v, g, beta)
    to = lambda u: torch.from_numpy(np.ascontiguousarray(u))
    # The layer's state is [dk][dv] and it scales q by 1/sqrt(dk) itself.
    ref_o, ref_S = tq.torch_recurrent_gated_delta_rule(
        to(q * math.sqrt(DK)), to(k), to(v), g=to(g), beta=to(beta), initial_state=to(S0.transpose(0, 1, 3, 2)),
        output_final_state=True, use_qk_l2norm_in_kernel=False)
    assert _rel(o, ref_o.double().numpy()) <= FP32_BAR
    assert _rel(S, ref_S.double().numpy().transpose(0, 1, 3, 2)) <= FP32_BAR


def test_epilogue_matches_the_gated_rms_norm():
    rng = np.random.default_rng(3)
    o = rng.normal(size=(5, H, DV)) * 0.05
    z = rng.normal(size=(5, H, DV))
    w = 1 + 0.1 * rng.normal(size=DV)
    norm = tq.Qwen3NextRMSNormGated(DV, eps=1e-6).double()
    with torch.no_grad():
        norm.weight.copy_(torch.from_numpy(w))
        ref = norm(torch.from_numpy(o).reshape(-1, DV), torch.from_numpy(z).reshape(-1, DV)).reshape(o.shape)
    assert _rel(M.epilogue(o, z, w), ref.double().numpy()) <= FP32_BAR


def test_layer_end_to_end(monkeypatch):
    """Zero history and zero state: the layer's forward over L rows equals the
    oracle's prologue, recurrence and epilogue over the same rows (the oracle's
    bf16 rounding switched off; the layer keeps fp64 operands)."""
    layer = _layer(4)
    B, L = 2, 11
    h = torch.randn(B, L, HID, dtype=torch.float64)
    _capture(monkeypatch)
    with torch.no_grad():
        ref = layer(h).reshape(B, L, H, DV).double().numpy()
    x, z, a, b = _raw(layer, h)
    monkeypatch.setattr(M, "bf16_round", lambda u: np.asarray(u, np.float64))
    q, k, v, g, beta = M.prologue(x, np.zeros((B, 3, x.shape[2])), layer.conv1d.weight[:, 0, :].detach().numpy(),
                                  a, b, layer.A_log.detach().numpy(), layer.dt_bias.detach().numpy(), HK, DK, H, DV)
    o, _ = oracle.prefill_seq(np.zeros((B, H, DV, DK)), q, k, v, g, beta)
    y = M.epilogue(o, z, layer.norm.weight.detach().numpy())
    assert _rel(y, ref) <= FP32_BAR
