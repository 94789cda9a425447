"""Independent reference points that pin the GDN-2 oracle (test infrastructure).

Each function here is written from its own textbook definition, not from the
GDN-2 oracle's code, so that agreement in a special case says something:

* ``kda_textbook``       Kimi Delta Attention: S <- (I - beta k k^T) Diag(alpha) S
                         + beta k v^T.  The pages state that GDN-2 recovers KDA
                         exactly when both gates collapse to one scalar
                         (aiexpert.news/pt, method paragraph).
* ``gdn_textbook``       Gated DeltaNet in the value-by-key convention
                         S' = a S (I - beta k k^T) + beta v k^T, o = S' q; GDN-2
                         reduces to it when the decay collapses as well
                         (needhelp.icu/de, section "Generalisierungshierarchie").
* ``deltanet_textbook``  DeltaNet written as "read, diff, write the delta":
                         S' = S - beta (S k - v) k^T (aixai.ru blog, linear-
                         attention section and FAQ on the delta rule).
* ``linear_attention_closed``  o_t = S0^T q_t + sum_{s<=t} (q_t . k_s) v_s, the
                         O(T^2) form of plain linear attention (aixai.ru blog,
                         linear-attention section: history folded into a
                         dk x dv state by outer products).
* ``decayed_linear_closed`` the same with a per-key-channel decay:
                         o_t = sum_c q_tc e^{G_tc} S0[c,:] +
                               sum_{s<=t} sum_c q_tc k_sc e^{G_tc - G_sc} v_s,
                         G the running sum of log alpha.

All inputs are float64 NumPy arrays of a single head: q, k [T, dk], v [T, dv],
state [dk, dv] unless the docstring says otherwise.
"""
from __future__ import annotations

import numpy as np


def kda_textbook(q, k, v, alpha, beta, S0):
    """alpha [T, dk], beta [T].  Returns (o [T, dv], S [dk, dv])."""
    T, dk = k.shape
    S = S0.copy()
    eye = np.eye(dk)
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        S = (eye - beta[t] * np.outer(k[t], k[t])) @ (np.diag(alpha[t]) @ S) \
            + beta[t] * np.outer(k[t], v[t])
        o[t] = S.T @ q[t]
    return o, S


def gdn_textbook(q, k, v, a, beta, S0):
    """Scalar decay a [T], beta [T]; the state is carried as M = S^T
    (dv x dk) in this function.  Returns (o [T, dv], S [dk, dv])."""
    T, dk = k.shape
    M = S0.T.copy()
    eye = np.eye(dk)
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        M = M @ (a[t] * (eye - beta[t] * np.outer(k[t], k[t]))) + beta[t] * np.outer(v[t], k[t])
        o[t] = M @ q[t]
    return o, M.T


def deltanet_textbook(q, k, v, beta, S0):
    """No decay.  State carried as M = S^T (dv x dk)."""
    T, _ = k.shape
    M = S0.T.copy()
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        read = M @ k[t]
        M = M - beta[t] * np.outer(read - v[t], k[t])
        o[t] = M @ q[t]
    return o, M.T


def linear_attention_closed(q, k, v, S0):
    T = q.shape[0]
    scores = q @ k.T                      # [T, T], (q_t . k_s)
    mask = np.tril(np.ones((T, T)))       # s <= t
    return (scores * mask) @ v + q @ S0


def decayed_linear_closed(q, k, v, alpha, S0):
    G = np.cumsum(np.log(alpha), axis=0)  # [T, dk]
    T, dk = q.shape
    o = np.zeros((T, v.shape[1]))
    for t in range(T):
        acc = (q[t] * np.exp(G[t])) @ S0
        for s in range(t + 1):
            acc = acc + np.sum(q[t] * k[s] * np.exp(G[t] - G[s])) * v[s]
        o[t] = acc
    return o
