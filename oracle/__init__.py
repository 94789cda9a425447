"""CPU oracle of the Gated DeltaNet-2 recurrence (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  It shares no code with the GPU library and the
GPU library never imports it.

``fwd`` and ``decode`` run the plain float64 token-by-token recurrence written
in C (``gdn2_oracle.c``); ``bwd`` runs its hand-derived reverse-mode
derivative, token by token from the last.  ``segment_map`` and
``segment_combine`` (NumPy, float64) give the affine state map of a run of
tokens and the exclusive scan that chains such maps.  Inputs are the stored
tensors (float32 or bf16), upcast to float64 exactly; outputs are float64
NumPy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn2_oracle.so")
_lib = None

RULES = {"R5": 0, "R1": 1}


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (host only, OpenMP)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall",
                        "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        lib.gdn2_oracle_fwd.restype = ctypes.c_int
        lib.gdn2_oracle_fwd.argtypes = [dp] * 7 + [ip] + [ctypes.c_int] * 7 + [dp, dp]
        lib.gdn2_oracle_decode.restype = ctypes.c_int
        lib.gdn2_oracle_decode.argtypes = [dp] * 7 + [ctypes.c_int] * 5 + [dp]
        lib.gdn2_oracle_bwd.restype = ctypes.c_int
        lib.gdn2_oracle_bwd.argtypes = ([dp] * 7 + [ip] + [ctypes.c_int] * 6 + [dp] * 9)
        lib.gdn2_oracle_max_threads.restype = ctypes.c_int
        lib.gdn2_oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _f64(x) -> np.ndarray:
    """Stored tensor (torch or numpy, any float dtype) -> contiguous float64."""
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads() -> int:
    return int(_load().gdn2_oracle_max_threads())


def set_threads(n: int) -> None:
    _load().gdn2_oracle_set_threads(int(n))


def fwd(q, k, v, alpha, b, w, S0=None, cu_seqlens=None, rule: str = "R5"):
    """Token-by-token forward.  Shapes [B,T,H,d]; S0 [N,H,dk,dv] or None.
    Returns (o [B,T,H,dv], S_final [N,H,dk,dv]) as float64 arrays."""
    q, k, v, alpha, b, w = (_f64(x) for x in (q, k, v, alpha, b, w))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.numpy() if hasattr(cu_seqlens, "numpy") else cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    else:
        cu, N, cu_p = None, B, None
    S0a = _f64(S0)
    o = np.zeros((B, T, H, dv), dtype=np.float64)
    Sf = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load().gdn2_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w),
                                 _ptr(S0a), cu_p, B, T, H, dk, dv, N, RULES[rule],
                                 _ptr(o), _ptr(Sf))
    if rc != 0:
        raise RuntimeError(f"gdn2_oracle_fwd failed with code {rc}")
    return o, Sf


def decode(q, k, v, alpha, b, w, S, rule: str = "R5"):
    """One decode step; inputs [N,H,d]; S [N,H,dk,dv] (not modified).
    Returns (o [N,H,dv], S_new [N,H,dk,dv]) as float64 arrays."""
    q, k, v, alpha, b, w = (_f64(x) for x in (q, k, v, alpha, b, w))
    N, H, dk = q.shape
    dv = v.shape[-1]
    Sn = _f64(S).copy()
    o = np.zeros((N, H, dv), dtype=np.float64)
    rc = _load().gdn2_oracle_decode(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w),
                                    _ptr(Sn), N, H, dk, dv, RULES[rule], _ptr(o))
    if rc != 0:
        raise RuntimeError(f"gdn2_oracle_decode failed with code {rc}")
    return o, Sn


def bwd(q, k, v, alpha, b, w, dout, S0=None, dS_final=None, cu_seqlens=None):
    """Gradients of the rule-0 forward: given dL/do [B,T,H,dv] and dL/dS_final
    [N,H,dk,dv] (None = zero), returns a dict of float64 arrays dq, dk, dv,
    dalpha, db, dw (each its input's shape) and dS0 [N,H,dk,dv]."""
    q, k, v, alpha, b, w, do = (_f64(x) for x in (q, k, v, alpha, b, w, dout))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if cu_seqlens is not None:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.numpy() if hasattr(cu_seqlens, "numpy") else cu_seqlens, dtype=np.int32))
        N = cu.shape[0] - 1
        cu_p = cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    else:
        cu, N, cu_p = None, B, None
    S0a, dSf = _f64(S0), _f64(dS_final)
    g = {name: np.zeros(x.shape, dtype=np.float64)
         for name, x in (("dq", q), ("dk", k), ("dv", v), ("dalpha", alpha), ("db", b), ("dw", w))}
    g["dS0"] = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load().gdn2_oracle_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w),
                                 _ptr(S0a), cu_p, B, T, H, dk, dv, N, _ptr(do), _ptr(dSf),
                                 _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dalpha"]),
                                 _ptr(g["db"]), _ptr(g["dw"]), _ptr(g["dS0"]))
    if rc != 0:
        raise RuntimeError(f"gdn2_oracle_bwd failed with code {rc}")
    return g


def _sequences(B, T, cu_seqlens):
    """(row, start, end) of every sequence: B rows of T tokens, or packed."""
    if cu_seqlens is None:
        return [(n, 0, T) for n in range(B)]
    cu = np.asarray(cu_seqlens.numpy() if hasattr(cu_seqlens, "numpy") else cu_seqlens, dtype=np.int64)
    return [(0, int(cu[i]), int(cu[i + 1])) for i in range(cu.shape[0] - 1)]


def segment_map(q, k, v, alpha, b, w, cu_seqlens=None):
    """Affine state map S_out = Phi S_in + Psi of every sequence (rule R5).

    Putting D = Diag(alpha) S and z = w (.) v - D^T (b (.) k) into
    S' = D + k z^T (the formal paragraph of the aixai.ru Gated DeltaNet-2
    blog, in this library's reading) gives, per token,
        S' = A S + k (w (.) v)^T,   A = (I - k (b (.) k)^T) Diag(alpha),
    so over a run of tokens Phi = A_last ... A_first and Psi is the state
    reached from zero.  Both are accumulated token by token in float64:
    Phi <- A Phi, Psi <- A Psi + k (w (.) v)^T, with A applied as its two
    factors.  Returns (Phi [N,H,dk,dk], Psi [N,H,dk,dv])."""
    q, k, v, alpha, b, w = (_f64(x) for x in (q, k, v, alpha, b, w))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    seqs = _sequences(B, T, cu_seqlens)
    Phi = np.zeros((len(seqs), H, dk, dk))
    Psi = np.zeros((len(seqs), H, dk, dv))
    for i, (n, s, e) in enumerate(seqs):
        P = np.broadcast_to(np.eye(dk), (H, dk, dk)).copy()
        Q = np.zeros((H, dk, dv))
        for t in range(s, e):
            kt, bt, at = k[n, t], b[n, t], alpha[n, t]           # [H, dk]
            for M in (P, Q):
                M *= at[:, :, None]                              # Diag(alpha) M
                M -= kt[:, :, None] * np.einsum("hi,hij->hj", bt * kt, M)[:, None, :]
            Q += kt[:, :, None] * (w[n, t] * v[n, t])[:, None, :]
        Phi[i], Psi[i] = P, Q
    return Phi, Psi


def segment_combine(Phi, Psi, S0=None):
    """Exclusive scan of consecutive segments' maps [G,H,..]: the state
    entering segment g, S_in[0] = S0 (zero if None), S_in[g+1] =
    Phi[g] S_in[g] + Psi[g].  Returns (S_in [G,H,dk,dv], S_final [H,dk,dv])."""
    Phi, Psi = _f64(Phi), _f64(Psi)
    G, H, dk, dv = Psi.shape
    S = np.zeros((H, dk, dv)) if S0 is None else _f64(S0).copy()
    S_in = np.zeros((G, H, dk, dv))
    for g in range(G):
        S_in[g] = S
        S = Phi[g] @ S + Psi[g]
    return S_in, S
