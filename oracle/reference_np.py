"""A second, literal NumPy transcription of the GDN-2 token recurrence
(test infrastructure, small shapes only).

It serves two purposes: a cross-check of the C oracle by an independent
implementation, and the "planted mistake" variants used to show that the pins
catch plausible errors.  The steps follow the formal paragraph of the aixai.ru
blog ("One scalar cannot decide two different questions"): decay the state per
key channel, read it with the erase-gated key, form the write-gated delta
value, write it along the key, then read the output after the update.

``mutation`` (for pin-power tests only) plants one mistake:
  "no_b_in_read"     read with the plain key instead of b (.) k
  "gated_write_key"  write along b (.) k instead of k
  "decay_after"      apply the decay after the write instead of before
  "read_before"      emit o from the state before the update
  "decay_value_axis" decay the value channels (columns) instead of key rows
  "transpose_read"   read with S instead of S^T (dk == dv only)
  "swap_gates"       use w on the key side and b on the value side
  "w_on_delta"       weight the whole delta by w (w (.) (v - read))
  "sign_write"       subtract the write instead of adding it
"""
from __future__ import annotations

import numpy as np


def step(S, q, k, v, alpha, b, w, rule="R5", mutation=None):
    """One token on one head; S [dk, dv] float64 (returned, not modified)."""
    if mutation == "swap_gates":
        b, w = w, b
    if mutation == "decay_value_axis":
        D = S * alpha[None, :]
    elif mutation == "decay_after":
        D = S.copy()
    else:
        D = S * alpha[:, None]
    e = b * k
    if rule == "R5":
        key = k if mutation == "no_b_in_read" else e
        read = (D @ key) if mutation == "transpose_read" else (D.T @ key)
        if mutation == "w_on_delta":
            z = w * (v - read)
        else:
            z = w * v - read
        wk = e if mutation == "gated_write_key" else k
        sgn = -1.0 if mutation == "sign_write" else 1.0
        Sn = D + sgn * np.outer(wk, z)
    elif rule == "R1":
        read = D.T @ k
        Sn = D - np.outer(e, read) + np.outer(k, w * v)
    else:
        raise ValueError(rule)
    if mutation == "decay_after":
        Sn = Sn * alpha[:, None]
    o = (S.T @ q) if mutation == "read_before" else (Sn.T @ q)
    return Sn, o


def fwd_head(q, k, v, alpha, b, w, S0, rule="R5", mutation=None):
    """One head, one sequence: q, k, alpha, b [T, dk]; v, w [T, dv]."""
    T = q.shape[0]
    S = S0.copy()
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        S, o[t] = step(S, q[t], k[t], v[t], alpha[t], b[t], w[t], rule, mutation)
    return o, S


def fwd(q, k, v, alpha, b, w, S0=None, rule="R5", mutation=None):
    """Batched [B, T, H, d] float64 arrays; S0 [B, H, dk, dv] or None."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    Sf = np.zeros((B, H, dk, dv))
    for n in range(B):
        for h in range(H):
            s0 = np.zeros((dk, dv)) if S0 is None else S0[n, h]
            o[n, :, h], Sf[n, h] = fwd_head(q[n, :, h], k[n, :, h], v[n, :, h], alpha[n, :, h],
                                            b[n, :, h], w[n, :, h], s0, rule, mutation)
    return o, Sf
