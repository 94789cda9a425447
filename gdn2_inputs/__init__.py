"""Seeded synthetic inputs for the GDN-2 forward and decode paths.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It draws random numbers and shapes them into tensors; it holds none
of the recurrence's arithmetic.

Recipe (every workload):
  * NumPy ``default_rng(seed)`` (PCG64), draws in float64, in the fixed order
    q, k, v, alpha-logit, b-logit, w-logit, S0.
  * q and k are L2-normalised per (token, head) in float64 before the cast:
    the pages place this normalisation outside the recurrence (Gated DeltaNet-2
    blog, aixai.ru, section "how it is implemented in practice").
  * v ~ N(0, 1); alpha = sigmoid(N(3, 1)) per key channel; b = sigmoid(N(0, 1))
    per key channel; w = sigmoid(N(0, 1)) per value channel; S0 ~ N(0, 0.1^2)
    (standard deviation 0.1) when a nonzero initial state is asked for.
  * The float64 draws are cast to the storage dtype with torch (bf16 is
    round-to-nearest-even).  Consumers read the stored tensors back; nobody
    uses the pre-rounding values.

All tensors are returned on the CPU, token-major ``[B, T, H, d]``.  The state is
``[N, H, dk, dv]`` float32 (key channel = row, value channel = column).
"""
from __future__ import annotations

import numpy as np
import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def _l2norm(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, 1e-30)


def _cast(x: np.ndarray, dtype: str) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(DTYPES[dtype]).contiguous()


def packed_lengths(seed: int, total: int = 32768, lo: int = 256, hi: int = 8192) -> list[int]:
    """Sequence lengths drawn uniformly from {lo..hi} until their sum reaches
    ``total``; the last one is truncated so the sum is exactly ``total``."""
    rng = np.random.default_rng(seed)
    lens: list[int] = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return lens


def cu_seqlens_from(lengths: list[int]) -> torch.Tensor:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return torch.from_numpy(cu)


def make_chunk_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype: str, seed: int,
                      s0: str | None = None, num_seqs: int | None = None,
                      scalar_beta: bool = False, alpha_mean: float = 3.0) -> dict:
    """Inputs of one chunked-forward call.

    ``s0``: None (no initial state), "zero" (explicit zeros) or "normal"
    (N(0, 0.1^2)).  ``num_seqs`` is the number of state slots (B for fixed
    length, the sequence count for packed input).  ``scalar_beta`` replaces
    b and w by one shared scalar beta = sigmoid(N(0,1)) per (batch, token,
    head), broadcast over channels (the collapsed-gate case).  ``alpha_mean``
    is the mean of the decay logit: 3 (the default) forgets within a few
    hundred tokens, 8 decays a channel by about e^-2.3 over 4096 tokens
    (a long-memory head).
    """
    rng = np.random.default_rng(seed)
    q = _l2norm(rng.standard_normal((B, T, H, dk)))
    k = _l2norm(rng.standard_normal((B, T, H, dk)))
    v = rng.standard_normal((B, T, H, dv))
    alpha = _sigmoid(rng.normal(alpha_mean, 1.0, (B, T, H, dk)))
    if scalar_beta:
        beta = _sigmoid(rng.standard_normal((B, T, H, 1)))
        b = np.broadcast_to(beta, (B, T, H, dk))
        w = np.broadcast_to(beta, (B, T, H, dv))
    else:
        b = _sigmoid(rng.standard_normal((B, T, H, dk)))
        w = _sigmoid(rng.standard_normal((B, T, H, dv)))
    n = B if num_seqs is None else num_seqs
    out = {
        "q": _cast(q, dtype), "k": _cast(k, dtype), "v": _cast(v, dtype),
        "alpha": _cast(alpha, dtype), "b": _cast(b, dtype), "w": _cast(w, dtype),
    }
    if s0 is None:
        out["S0"] = None
    elif s0 == "zero":
        out["S0"] = torch.zeros((n, H, dk, dv), dtype=torch.float32)
    elif s0 == "normal":
        out["S0"] = torch.from_numpy(rng.normal(0.0, 0.1, (n, H, dk, dv))).float().contiguous()
    else:
        raise ValueError(f"unknown s0 mode {s0!r}")
    return out


def make_strong_decay_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype: str, seed: int,
                             s0: str | None = None, num_seqs: int | None = None,
                             logit_mean: float = -2.0, logit_std: float = 2.0,
                             tiny_frac: float = 0.01, tiny: float = 1e-4, zero_frac: float = 0.01,
                             alpha_min: float = 0.0) -> dict:
    """Inputs of one chunked-forward call with strong and degenerate decay:
    as make_chunk_inputs, but alpha = sigmoid(N(logit_mean, logit_std^2))
    per key channel, then a fraction ``tiny_frac`` of the (token, head,
    channel) entries set to ``tiny`` and a fraction ``zero_frac`` set to 0
    exactly (drawn after everything else, from the same generator), and
    alpha raised to at least ``alpha_min``."""
    out = make_chunk_inputs(B, T, H, dk, dv, dtype, seed, s0=s0, num_seqs=num_seqs)
    rng = np.random.default_rng(seed + 104729)
    alpha = _sigmoid(rng.normal(logit_mean, logit_std, (B, T, H, dk)))
    u = rng.random((B, T, H, dk))
    alpha = np.where(u < tiny_frac, tiny, alpha)
    alpha = np.where((u >= tiny_frac) & (u < tiny_frac + zero_frac), 0.0, alpha)
    out["alpha"] = _cast(np.maximum(alpha, alpha_min), dtype)
    return out


def make_bwd_grads(B: int, T: int, H: int, dk: int, dv: int, dtype: str, seed: int,
                   num_seqs: int | None = None, with_dS: bool = True) -> dict:
    """Incoming gradients of one backward call: dL/do ~ N(0, 1) [B, T, H, dv]
    in ``dtype`` and dL/dS_final ~ N(0, 1) [N, H, dk, dv] float32 (None when
    ``with_dS`` is False)."""
    rng = np.random.default_rng(seed + 7919)
    n = B if num_seqs is None else num_seqs
    dS = torch.from_numpy(rng.standard_normal((n, H, dk, dv))).float().contiguous() if with_dS else None
    return {"dout": _cast(rng.standard_normal((B, T, H, dv)), dtype), "dS_final": dS}


def make_layer_inputs(B: int, T: int, H: int, dk: int, dv: int, dtype: str, seed: int,
                      s0: str | None = None, scalar_beta: bool = False, strong_decay: bool = False,
                      neg_inf_frac: float = 0.0) -> dict:
    """Raw layer inputs of one chunked-forward call in layer-prep mode: q and
    k not normalised (N(0,1) times a per-row scale in [0.5, 4]), v ~ N(0,1),
    gate logits b, w ~ N(0,1) (one shared logit per (batch, token, head) with
    ``scalar_beta``, then shaped [B, T, H]), and the natural-log decay
    log(sigmoid(N(3,1))) per key channel, always float32.  The recurrence
    inputs these stand for have the same distributions as make_chunk_inputs.
    With ``strong_decay`` the log-decay is log(sigmoid(N(-2, 2^2))) floored
    at -20, with 1% of the entries at -20 exactly, and a fraction
    ``neg_inf_frac`` at -inf (alpha = 0); these are drawn after everything
    else.
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk)) * rng.uniform(0.5, 4.0, (B, T, H, 1))
    k = rng.standard_normal((B, T, H, dk)) * rng.uniform(0.5, 4.0, (B, T, H, 1))
    v = rng.standard_normal((B, T, H, dv))
    log_alpha = np.log(_sigmoid(rng.normal(3.0, 1.0, (B, T, H, dk))))
    if scalar_beta:
        b = w = rng.standard_normal((B, T, H))
    else:
        b = rng.standard_normal((B, T, H, dk))
        w = rng.standard_normal((B, T, H, dv))
    out = {
        "q": _cast(q, dtype), "k": _cast(k, dtype), "v": _cast(v, dtype),
        "alpha": _cast(log_alpha, "f32"), "b": _cast(b, dtype), "w": _cast(w, dtype),
    }
    if s0 is None:
        out["S0"] = None
    elif s0 == "normal":
        out["S0"] = torch.from_numpy(rng.normal(0.0, 0.1, (B, H, dk, dv))).float().contiguous()
    else:
        raise ValueError(f"unknown s0 mode {s0!r}")
    if strong_decay:
        r2 = np.random.default_rng(seed + 104729)
        la = np.maximum(np.log(_sigmoid(r2.normal(-2.0, 2.0, (B, T, H, dk)))), -20.0)
        u = r2.random((B, T, H, dk))
        la = np.where(u < 0.01, -20.0, la)
        la = np.where((u >= 0.01) & (u < 0.01 + neg_inf_frac), -np.inf, la)
        out["alpha"] = _cast(la, "f32")
    return out


def make_decode_inputs(N: int, H: int, dk: int, dv: int, dtype: str, seed: int,
                       steps: int) -> dict:
    """``steps`` distinct single-token inputs ``[steps, N, H, d]`` plus a state
    ``S ~ N(0, 0.1^2)`` of shape ``[N, H, dk, dv]`` float32."""
    rng = np.random.default_rng(seed)
    q = _l2norm(rng.standard_normal((steps, N, H, dk)))
    k = _l2norm(rng.standard_normal((steps, N, H, dk)))
    v = rng.standard_normal((steps, N, H, dv))
    alpha = _sigmoid(rng.normal(3.0, 1.0, (steps, N, H, dk)))
    b = _sigmoid(rng.standard_normal((steps, N, H, dk)))
    w = _sigmoid(rng.standard_normal((steps, N, H, dv)))
    S = rng.normal(0.0, 0.1, (N, H, dk, dv))
    return {
        "q": _cast(q, dtype), "k": _cast(k, dtype), "v": _cast(v, dtype),
        "alpha": _cast(alpha, dtype), "b": _cast(b, dtype), "w": _cast(w, dtype),
        "S": torch.from_numpy(S).float().contiguous(),
    }


# The five workloads (shapes, dtypes, seeds), named by what they are: a tiny
# and a small float32 case the oracle finishes in seconds, the 1.3B-scale
# layer (8 x 4096 tokens x 16 heads, d = 128, bf16), 32768 packed tokens of
# mixed lengths (from ``packed_lengths(3)``; its sweep uses fixed-length
# batches with B * T = 32768), and a decode step of 256 sequences x 16 heads.
WORKLOADS = {
    "tiny_1x64x1_d16": dict(B=1, H=1, T=64, dk=16, dv=16, chunk=16, dtype="f32", seed=0, s0="zero"),
    "small_2x512x4_d64": dict(B=2, H=4, T=512, dk=64, dv=64, chunk=64, dtype="f32", seed=1, s0="normal"),
    "layer_8x4096x16_d128": dict(B=8, H=16, T=4096, dk=128, dv=128, chunk=64, dtype="bf16", seed=2, s0=None),
    "packed_32768x16_d128": dict(B=1, H=16, T=32768, dk=128, dv=128, chunk=64, dtype="bf16", seed=3, s0=None,
                                 packed=True),
    "decode_256x16_d128": dict(N=256, H=16, dk=128, dv=128, dtype="bf16", seed=4, steps=16),
}

SWEEP_T = (2048, 4096, 8192, 16384, 32768)
