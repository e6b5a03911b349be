"""ctypes front end of the fp64 C oracle (``gdn_oracle.c``).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it; the product path never does.

Arrays are numpy; every input is widened to float64 exactly (bf16 and fp32
values are exactly representable in fp64) before the C code sees it.

Layouts follow the C file:  S [B][H][dv][dk];  q, k [B][L][H][dk];
v [B][L][H][dv];  g, beta [B][L][H];  o [B][L][H][dv].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def lib_path() -> str:
    return _LIB


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, strict IEEE: no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", *compile_flags(), _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def compile_flags() -> list[str]:
    return ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off"]


def bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Declare the C entry points' signatures on a loaded oracle library."""
    dp = ctypes.POINTER(ctypes.c_double)
    ip = ctypes.POINTER(ctypes.c_int)
    lib.oracle_gdn_seq.restype = ctypes.c_int
    lib.oracle_gdn_seq.argtypes = [ctypes.c_int] * 5 + [dp] * 6 + [ip, dp, dp]
    lib.oracle_gdn_chunked.restype = ctypes.c_int
    lib.oracle_gdn_chunked.argtypes = [ctypes.c_int] * 6 + [dp] * 7
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = bind(ctypes.CDLL(_LIB))
    return _lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a CPU torch tensor: take its exact values
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _dims(S, q, v, g):
    B, H, dv, dk = S.shape
    L = q.shape[1]
    assert q.shape == (B, L, H, dk), q.shape
    assert v.shape == (B, L, H, dv), v.shape
    assert g.shape == (B, L, H), g.shape
    return B, H, dk, dv, L


def gdn_seq(S0, q, k, v, g, beta, keep=None, want_o=True, want_state=True):
    """Run the sequential recurrence; returns (o, S_keep) as float64 arrays.

    ``keep`` (int array [B] or None) selects the returned state S_keep[b] =
    S_{keep[b]}; keep[b] == 0 returns S0 itself, byte for byte.
    """
    S0, q, k, v, g, beta = map(_f64, (S0, q, k, v, g, beta))
    B, H, dk, dv, L = _dims(S0, q, v, g)
    assert k.shape == q.shape and beta.shape == g.shape
    o = np.empty((B, L, H, dv), np.float64) if want_o else None
    Sout = np.empty_like(S0) if want_state else None
    kp = None
    if keep is not None:
        keep_arr = np.ascontiguousarray(np.asarray(keep, dtype=np.int32).reshape(B))
        kp = keep_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int))
    rc = _load().oracle_gdn_seq(B, H, dk, dv, L, _ptr(S0), _ptr(q), _ptr(k), _ptr(v),
                                _ptr(g), _ptr(beta), kp, _ptr(o), _ptr(Sout))
    if rc != 0:
        raise ValueError("oracle_gdn_seq rejected its arguments")
    return o, Sout


def verify(S0, q, k, v, g, beta):
    """Outputs o_1..o_T of a verify block; the state is not advanced."""
    o, _ = gdn_seq(S0, q, k, v, g, beta, want_state=False)
    return o


def commit(S0, q, k, v, g, beta, n):
    """State after the first n[b] rows of the block, per instance b."""
    _, S = gdn_seq(S0, q, k, v, g, beta, keep=n, want_o=False)
    return S


def prefill_seq(S0, q, k, v, g, beta):
    """All outputs and the final state of a prompt, token by token."""
    return gdn_seq(S0, q, k, v, g, beta)


def prefill_chunked(S0, q, k, v, g, beta, chunk):
    """The fp64 UT/WY chunk form; returns (o, S_final)."""
    S = _f64(S0).copy()
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    B, H, dk, dv, L = _dims(S, q, v, g)
    o = np.empty((B, L, H, dv), np.float64)
    rc = _load().oracle_gdn_chunked(B, H, dk, dv, L, int(chunk), _ptr(S), _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(g), _ptr(beta), _ptr(o))
    if rc != 0:
        raise ValueError("oracle_gdn_chunked rejected its arguments")
    return o, S
