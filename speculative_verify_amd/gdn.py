"""Python binding of libgdn (include/gdn.h), by ctypes.

Argument marshalling only: every function checks that the torch tensors it is
handed match the layouts the C ABI documents, passes raw device pointers and
the current HIP stream, and raises GdnError on a non-zero status.  All
arithmetic happens in libgdn's HIP kernels.  There is no fallback: if
libgdn.so is missing the import fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn.so")

GDN_IN_F32 = 0
GDN_IN_BF16 = 1
GDN_T_MAX = 16
GDN_PREFILL_CHUNK = 64
GDN_REC_NO_BLOCK = 1
GDN_REC_N_RANGE = 2
GDN_REC_SHAPE = 4

EXPORTED = (
    "gdn_block_record_bytes",
    "gdn_verify_block",
    "gdn_commit",
    "gdn_commit_verify",
    "gdn_record_status",
    "gdn_prefill_workspace_bytes",
    "gdn_prefill_chunked",
    "gdn_accept_workspace_bytes",
    "gdn_accept_sampled_noalloc",
    "gdn_accept_noalloc_max_bytes",
    "gdn_accept_greedy",
    "gdn_accept_sampled",
    "gdn_history_rewind",
    "gdn_attn_workspace_bytes",
    "gdn_attn_verify",
    "gdn_mixer_verify",
    "gdn_mixer_commit_verify",
    "gdn_strerror",
)
GDN_HISTORY_MAX = 16


class GdnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status} ({strerror(status)})")
        self.status = status


class gdn_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("dk", ctypes.c_int32),
                ("dv", ctypes.c_int32)]


class gdn_accept_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("V", ctypes.c_int32)]


class gdn_mixer_inputs(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("history", ctypes.c_void_p), ("conv_w", ctypes.c_void_p),
                ("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("A_log", ctypes.c_void_p),
                ("dt_bias", ctypes.c_void_p), ("z", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
                ("Hk", ctypes.c_int32)]


class gdn_attn_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("Lmax", ctypes.c_int32)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m speculative_verify_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    sp = ctypes.POINTER(gdn_shape)
    lib.gdn_block_record_bytes.restype = sz
    lib.gdn_block_record_bytes.argtypes = [sp, i32, ctypes.c_int]
    lib.gdn_verify_block.restype = ctypes.c_int
    lib.gdn_verify_block.argtypes = [vp] * 6 + [i32, ctypes.c_int, sp, vp, vp, sz, vp]
    lib.gdn_commit.restype = ctypes.c_int
    lib.gdn_commit.argtypes = [vp, vp, vp, vp, sp, vp]
    lib.gdn_commit_verify.restype = ctypes.c_int
    lib.gdn_commit_verify.argtypes = [vp] * 9 + [i32, ctypes.c_int, sp, vp, vp, sz, vp]
    lib.gdn_record_status.restype = ctypes.c_int
    lib.gdn_record_status.argtypes = [vp, sp, ctypes.POINTER(i32), vp]
    lib.gdn_prefill_workspace_bytes.restype = sz
    lib.gdn_prefill_workspace_bytes.argtypes = [sp, i32, i32]
    lib.gdn_prefill_chunked.restype = ctypes.c_int
    lib.gdn_prefill_chunked.argtypes = [vp] * 6 + [i32, i32, ctypes.c_int, sp, vp, vp, sz, vp]
    ap = ctypes.POINTER(gdn_accept_shape)
    lib.gdn_accept_workspace_bytes.restype = sz
    lib.gdn_accept_workspace_bytes.argtypes = [ap, i32]
    lib.gdn_accept_greedy.restype = ctypes.c_int
    lib.gdn_accept_greedy.argtypes = [vp, ctypes.c_int, vp, ap, vp, vp, vp, sz, vp]
    lib.gdn_accept_sampled.restype = ctypes.c_int
    lib.gdn_accept_sampled.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, ctypes.c_float, ap, vp, vp, vp, sz, vp]
    lib.gdn_accept_sampled_noalloc.restype = ctypes.c_int
    lib.gdn_accept_sampled_noalloc.argtypes = [vp, vp, ctypes.c_int, vp, vp, vp, ctypes.c_float, ap, vp, vp, vp]
    lib.gdn_accept_noalloc_max_bytes.restype = sz
    lib.gdn_accept_noalloc_max_bytes.argtypes = []
    lib.gdn_history_rewind.restype = ctypes.c_int
    lib.gdn_history_rewind.argtypes = [vp, vp, vp, i32, i32, i32, i32, ctypes.c_int, vp]
    mp = ctypes.POINTER(gdn_mixer_inputs)
    lib.gdn_mixer_verify.restype = ctypes.c_int
    lib.gdn_mixer_verify.argtypes = [vp, mp, i32, sp, vp, vp, sz, vp]
    lib.gdn_mixer_commit_verify.restype = ctypes.c_int
    lib.gdn_mixer_commit_verify.argtypes = [vp, vp, vp, vp, mp, i32, sp, vp, vp, sz, vp]
    tp = ctypes.POINTER(gdn_attn_shape)
    lib.gdn_attn_workspace_bytes.restype = sz
    lib.gdn_attn_workspace_bytes.argtypes = [tp, i32]
    lib.gdn_attn_verify.restype = ctypes.c_int
    lib.gdn_attn_verify.argtypes = [vp] * 6 + [i32, ctypes.c_float, tp, vp, vp, sz, vp]
    lib.gdn_strerror.restype = ctypes.c_char_p
    lib.gdn_strerror.argtypes = [ctypes.c_int]
    return lib


lib = _load()


def strerror(status: int) -> str:
    return lib.gdn_strerror(int(status)).decode()


def _dt(x: torch.Tensor) -> int:
    if x.dtype == torch.bfloat16:
        return GDN_IN_BF16
    if x.dtype == torch.float32:
        return GDN_IN_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {x.dtype}")


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        if not x.is_contiguous():
            raise ValueError("tensors must be contiguous")
        return ctypes.c_void_p(x.data_ptr())
    return ctypes.c_void_p(int(x))


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _shape_of(S: torch.Tensor) -> gdn_shape:
    if S.dtype != torch.float32 or S.dim() != 4:
        raise ValueError("S must be fp32 [B][H][dv][dk]")
    B, H, dv, dk = S.shape
    return gdn_shape(B, H, dk, dv)


def _check_rows(shp: gdn_shape, q, k, v, g, beta, o):
    B, H, dk, dv = shp.B, shp.H, shp.dk, shp.dv
    T = q.shape[1]
    want = {"q": (q, (B, T, H, dk)), "k": (k, (B, T, H, dk)), "v": (v, (B, T, H, dv)),
            "g": (g, (B, T, H)), "beta": (beta, (B, T, H)), "o": (o, (B, T, H, dv))}
    for name, (x, shape) in want.items():
        if tuple(x.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(x.shape)}, expected {shape}")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share one dtype")
    for name, x in (("g", g), ("beta", beta), ("o", o)):
        if x.dtype != torch.float32:
            raise TypeError(f"{name} must be float32")
    return T


def gdn_block_record_bytes(B: int, H: int, dk: int, dv: int, T: int, dtype) -> int:
    dt = _dt(torch.empty(0, dtype=dtype))
    return int(lib.gdn_block_record_bytes(ctypes.byref(gdn_shape(B, H, dk, dv)), T, dt))


def new_record(S: torch.Tensor, T: int, dtype) -> torch.Tensor:
    """A zero-filled device buffer sized for blocks of T rows of S's shape."""
    B, H, dv, dk = S.shape
    n = gdn_block_record_bytes(B, H, dk, dv, T, dtype)
    if n == 0:
        raise ValueError("invalid shape, T or dtype for a block record")
    return torch.zeros(n, dtype=torch.uint8, device=S.device)


def gdn_verify_block(S, q, k, v, g, beta, o, record, stream=None) -> None:
    """o[:] = outputs of the T-row block (q, k, v, g, beta) from checkpoint S; the
    record becomes the pending block.  S is not modified."""
    shp = _shape_of(S)
    T = _check_rows(shp, q, k, v, g, beta, o)
    rc = lib.gdn_verify_block(_ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), T,
                              _dt(q), ctypes.byref(shp), _ptr(o), _ptr(record),
                              record.numel() * record.element_size(), _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_verify_block")


def gdn_commit(S, record, n_accepted, pos=None, stream=None) -> None:
    """S <- state after the first n_accepted[b] rows of the pending block
    (device int32 [B]); pos[b] += n_accepted[b] when pos is given."""
    shp = _shape_of(S)
    for name, x in (("n_accepted", n_accepted), ("pos", pos)):
        if x is not None and (x.dtype != torch.int32 or tuple(x.shape) != (shp.B,)):
            raise ValueError(f"{name} must be int32 [{shp.B}]")
    rc = lib.gdn_commit(_ptr(S), _ptr(record), _ptr(n_accepted), _ptr(pos), ctypes.byref(shp),
                        _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_commit")


def gdn_commit_verify(S, record_prev, n_accepted, q, k, v, g, beta, o, record_next, pos=None,
                      stream=None) -> None:
    """gdn_commit(S, record_prev, n_accepted, pos) then gdn_verify_block(S, q, k, v,
    g, beta, o, record_next), in one pass over the state."""
    shp = _shape_of(S)
    T = _check_rows(shp, q, k, v, g, beta, o)
    for name, x in (("n_accepted", n_accepted), ("pos", pos)):
        if x is not None and (x.dtype != torch.int32 or tuple(x.shape) != (shp.B,)):
            raise ValueError(f"{name} must be int32 [{shp.B}]")
    rc = lib.gdn_commit_verify(_ptr(S), _ptr(record_prev), _ptr(n_accepted), _ptr(pos), _ptr(q), _ptr(k),
                               _ptr(v), _ptr(g), _ptr(beta), T, _dt(q), ctypes.byref(shp), _ptr(o),
                               _ptr(record_next), record_next.numel() * record_next.element_size(),
                               _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_commit_verify")


def gdn_record_status(record, S, stream=None) -> list[int]:
    """Per-instance GDN_REC_* error bits of the last commit (synchronising)."""
    shp = _shape_of(S)
    out = (ctypes.c_int32 * shp.B)()
    rc = lib.gdn_record_status(_ptr(record), ctypes.byref(shp), out, _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_record_status")
    return list(out)


def gdn_prefill_workspace_bytes(S, L: int, chunk: int = GDN_PREFILL_CHUNK) -> int:
    return int(lib.gdn_prefill_workspace_bytes(ctypes.byref(_shape_of(S)), L, chunk))


def gdn_prefill_chunked(S, q, k, v, g, beta, o, chunk: int = GDN_PREFILL_CHUNK, ws=None,
                        stream=None) -> None:
    """Run the prompt (q, k, v, g, beta) through the recurrence: o[:] = all outputs,
    S advanced in place to the final state.  ``ws`` is the optional workspace of
    gdn_prefill_workspace_bytes bytes; when None it is allocated here (device
    memory only; all work runs in libgdn's kernels)."""
    shp = _shape_of(S)
    L = _check_rows(shp, q, k, v, g, beta, o)
    if ws is None:
        need = int(lib.gdn_prefill_workspace_bytes(ctypes.byref(shp), L, chunk))
        if need > 0:
            ws = torch.empty(need, dtype=torch.uint8, device=S.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    rc = lib.gdn_prefill_chunked(_ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), L,
                                 chunk, _dt(q), ctypes.byref(shp), _ptr(o), _ptr(ws), ws_bytes,
                                 _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_prefill_chunked")


def _accept_shape(target_logits) -> gdn_accept_shape:
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B][T][V]")
    B, T, V = target_logits.shape
    return gdn_accept_shape(B, T, V)


def _check_accept(shp, draft_tokens, n_out, next_token):
    B, T = shp.B, shp.T
    if T > 1 and (draft_tokens is None or tuple(draft_tokens.shape) != (B, T - 1)
                  or draft_tokens.dtype != torch.int32):
        raise ValueError("draft_tokens must be int32 [B][T-1]")
    for name, x in (("n_out", n_out), ("next_token", next_token)):
        if tuple(x.shape) != (B,) or x.dtype != torch.int32:
            raise ValueError(f"{name} must be int32 [B]")


def gdn_accept_workspace_bytes(target_logits, sampled: bool) -> int:
    return int(lib.gdn_accept_workspace_bytes(ctypes.byref(_accept_shape(target_logits)), int(bool(sampled))))


def _accept_ws(shp, sampled, device, ws):
    if ws is None:
        need = int(lib.gdn_accept_workspace_bytes(ctypes.byref(shp), int(sampled)))
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def gdn_accept_greedy(target_logits, draft_tokens, n_out, next_token, ws=None, stream=None) -> None:
    """Greedy acceptance of one verify block per sequence, on the device: n_out[b]
    = 1 + drafts kept, next_token[b] = the emitted (correction or bonus) token.
    ``ws`` is the workspace of gdn_accept_workspace_bytes(target_logits, False)
    bytes; when None it is allocated here (device memory only)."""
    shp = _accept_shape(target_logits)
    _check_accept(shp, draft_tokens, n_out, next_token)
    ws, nb = _accept_ws(shp, False, target_logits.device, ws)
    rc = lib.gdn_accept_greedy(_ptr(target_logits), _dt(target_logits), _ptr(draft_tokens), ctypes.byref(shp),
                               _ptr(n_out), _ptr(next_token), _ptr(ws), nb, _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_accept_greedy")


def gdn_accept_sampled(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature, n_out,
                       next_token, ws=None, stream=None) -> None:
    """Exact speculative sampling of one verify block per sequence, on the device
    (see gdn_accept_sampled in include/gdn.h)."""
    shp = _accept_shape(target_logits)
    _check_accept(shp, draft_tokens, n_out, next_token)
    B, T, V = shp.B, shp.T, shp.V
    if T > 1:
        if tuple(draft_logits.shape) != (B, T - 1, V) or draft_logits.dtype != target_logits.dtype:
            raise ValueError("draft_logits must be [B][T-1][V] in the target logits' dtype")
        if tuple(u_accept.shape) != (B, T - 1) or u_accept.dtype != torch.float32:
            raise ValueError("u_accept must be float32 [B][T-1]")
    if tuple(u_sample.shape) != (B,) or u_sample.dtype != torch.float32:
        raise ValueError("u_sample must be float32 [B]")
    ws, nb = _accept_ws(shp, True, target_logits.device, ws)
    rc = lib.gdn_accept_sampled(_ptr(target_logits), _ptr(draft_logits if T > 1 else None), _dt(target_logits),
                                _ptr(draft_tokens if T > 1 else None), _ptr(u_accept if T > 1 else None),
                                _ptr(u_sample), float(temperature), ctypes.byref(shp), _ptr(n_out),
                                _ptr(next_token), _ptr(ws), nb, _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_accept_sampled")


def gdn_accept_sampled_noalloc(target_logits, draft_logits, draft_tokens, u_accept, u_sample, temperature, n_out,
                               next_token, stream=None) -> None:
    """gdn_accept_sampled with the library's own per-device scratch instead of a
    workspace: allocates nothing (see gdn_accept_sampled_noalloc in
    include/gdn.h; calls that overlap on one device race)."""
    shp = _accept_shape(target_logits)
    _check_accept(shp, draft_tokens, n_out, next_token)
    B, T, V = shp.B, shp.T, shp.V
    if T > 1:
        if tuple(draft_logits.shape) != (B, T - 1, V) or draft_logits.dtype != target_logits.dtype:
            raise ValueError("draft_logits must be [B][T-1][V] in the target logits' dtype")
        if tuple(u_accept.shape) != (B, T - 1) or u_accept.dtype != torch.float32:
            raise ValueError("u_accept must be float32 [B][T-1]")
    if tuple(u_sample.shape) != (B,) or u_sample.dtype != torch.float32:
        raise ValueError("u_sample must be float32 [B]")
    rc = lib.gdn_accept_sampled_noalloc(_ptr(target_logits), _ptr(draft_logits if T > 1 else None),
                                        _dt(target_logits), _ptr(draft_tokens if T > 1 else None),
                                        _ptr(u_accept if T > 1 else None), _ptr(u_sample), float(temperature),
                                        ctypes.byref(shp), _ptr(n_out), _ptr(next_token), _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_accept_sampled_noalloc")


def gdn_history_rewind(history, rows, n, stream=None) -> None:
    """history [B][W][C] (in place) becomes the last W rows of [history; rows[:, :n]]
    per sequence; rows [B][T][C] in history's dtype; n int32 [B] on the device."""
    if history.dim() != 3 or rows.dim() != 3:
        raise ValueError("history must be [B][W][C] and rows [B][T][C]")
    B, W, C = history.shape
    if rows.shape[0] != B or rows.shape[2] != C or rows.dtype != history.dtype:
        raise ValueError("rows must be [B][T][C] in history's dtype")
    if tuple(n.shape) != (B,) or n.dtype != torch.int32:
        raise ValueError("n must be int32 [B]")
    rc = lib.gdn_history_rewind(_ptr(history), _ptr(rows), _ptr(n), B, W, rows.shape[1], C, _dt(history),
                                _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_history_rewind")


def _attn_shape(q, k_cache) -> gdn_attn_shape:
    if q.dim() != 4 or k_cache.dim() != 4:
        raise ValueError("q must be [B][T][Hq][d] and k_cache [B][Lmax][Hkv][d]")
    B, T, Hq, d = q.shape
    _, Lmax, Hkv, dk = k_cache.shape
    if dk != d or k_cache.shape[0] != B:
        raise ValueError("k_cache must be [B][Lmax][Hkv][d] with q's B and d")
    return gdn_attn_shape(B, Hq, Hkv, d, Lmax)


def gdn_attn_workspace_bytes(q, k_cache) -> int:
    return int(lib.gdn_attn_workspace_bytes(ctypes.byref(_attn_shape(q, k_cache)), q.shape[1]))


def gdn_attn_verify(q, k_new, v_new, k_cache, v_cache, ctx, o, scale=None, ws=None, stream=None) -> None:
    """Attention of a verify block (see gdn_attn_verify in include/gdn.h): o[:] =
    outputs, the block's keys and values written into the caches at ctx .. ctx+T-1.
    ``scale`` defaults to 1/sqrt(d); ``ws`` is the workspace of
    gdn_attn_workspace_bytes bytes (allocated here when None, device memory only)."""
    shp = _attn_shape(q, k_cache)
    B, T, Hq, d = q.shape
    want = {"k_new": (k_new, (B, T, shp.Hkv, d)), "v_new": (v_new, (B, T, shp.Hkv, d)),
            "v_cache": (v_cache, tuple(k_cache.shape))}
    for name, (x, shape) in want.items():
        if tuple(x.shape) != shape or x.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be bf16 {shape}")
    if q.dtype != torch.bfloat16 or k_cache.dtype != torch.bfloat16:
        raise ValueError("q and the caches must be bf16")
    if tuple(ctx.shape) != (B,) or ctx.dtype != torch.int32:
        raise ValueError("ctx must be int32 [B]")
    if tuple(o.shape) != (B, T, Hq, d) or o.dtype != torch.float32:
        raise ValueError("o must be float32 [B][T][Hq][d]")
    if scale is None:
        scale = 1.0 / float(d) ** 0.5
    if ws is None:
        need = int(lib.gdn_attn_workspace_bytes(ctypes.byref(shp), T))
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    nb = ws.numel() * ws.element_size()
    rc = lib.gdn_attn_verify(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(ctx), T,
                             float(scale), ctypes.byref(shp), _ptr(o), _ptr(ws), nb, _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_attn_verify")


def _mixer_struct(S, m, T):
    """The C struct of a MixerInputs (speculative_verify_amd.inputs), after shape checks."""
    B, H, dv, dk = S.shape
    cdim = 2 * m.Hk * dk + H * dv
    want = {"x": (m.x, (B, T, cdim), torch.bfloat16), "history": (m.history, (B, 3, cdim), torch.bfloat16),
            "conv_w": (m.conv_w, (cdim, 4), torch.float32), "a": (m.a, (B, T, H), torch.float32),
            "b": (m.b, (B, T, H), torch.float32), "A_log": (m.A_log, (H,), torch.float32),
            "dt_bias": (m.dt_bias, (H,), torch.float32), "z": (m.z, (B, T, H, dv), torch.bfloat16),
            "norm_w": (m.norm_w, (dv,), torch.float32)}
    for name, (x, shape, dt) in want.items():
        if tuple(x.shape) != shape or x.dtype != dt:
            raise ValueError(f"{name} must be {dt} {shape}")
    return gdn_mixer_inputs(*(ctypes.c_void_p(getattr(m, f).data_ptr()) for f in
                              ("x", "history", "conv_w", "a", "b", "A_log", "dt_bias", "z", "norm_w")), m.Hk)


def gdn_mixer_verify(S, m, y, record, stream=None) -> None:
    """The verify with the GDN mixer around it (see gdn_mixer_verify in
    include/gdn.h): y[:] = gated, normalised outputs; the record as for
    gdn_verify_block."""
    T = m.x.shape[1]
    shp = _shape_of(S)
    mi = _mixer_struct(S, m, T)
    if tuple(y.shape) != (shp.B, T, shp.H, shp.dv) or y.dtype != torch.float32:
        raise ValueError("y must be float32 [B][T][H][dv]")
    rc = lib.gdn_mixer_verify(_ptr(S), ctypes.byref(mi), T, ctypes.byref(shp), _ptr(y), _ptr(record),
                              record.numel() * record.element_size(), _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_mixer_verify")


def gdn_mixer_commit_verify(S, record_prev, n_accepted, m, y, record_next, pos=None, stream=None) -> None:
    """Commit of record_prev at n_accepted, then the mixer verify of the next block."""
    T = m.x.shape[1]
    shp = _shape_of(S)
    mi = _mixer_struct(S, m, T)
    if tuple(y.shape) != (shp.B, T, shp.H, shp.dv) or y.dtype != torch.float32:
        raise ValueError("y must be float32 [B][T][H][dv]")
    rc = lib.gdn_mixer_commit_verify(_ptr(S), _ptr(record_prev), _ptr(n_accepted), _ptr(pos), ctypes.byref(mi), T,
                                     ctypes.byref(shp), _ptr(y), _ptr(record_next),
                                     record_next.numel() * record_next.element_size(), _stream(stream))
    if rc != 0:
        raise GdnError(rc, "gdn_mixer_commit_verify")
