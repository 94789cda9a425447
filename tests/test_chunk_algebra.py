"""CPU design checks of the chunkwise algebra the GPU kernels implement,
written out in float64 NumPy from the derivation and compared with the
token-by-token oracle (no GPU, no code shared with the kernels).

* The forward's chunk form: per chunk of C tokens, with g the cumulative
  ln(alpha) from the chunk start, A = strict_lower(E Khat^T), T = (I + A)^-1,
  W = T E, Ut = T U, Z = Ut - W S, O = Qchk S + lower(Qchk Khat^T) Z,
  S' = Diag(gamma_C) S + Kbar^T Z (the chunkwise WY form with the erase gate
  inside the key products and the write gate inside the delta values:
  aixai.ru blog, section on how the method is implemented in practice).
* The decay factorisation of the kernels: every factor e^{g_t - g_s} built
  from sums of log decays per 16-token sub-block (row to its sub-block's
  start, key to its sub-block's end, the sub-blocks in between), diagonal
  blocks pair by pair with running products of the alphas when a sub-block
  decays by more than 2^-64, with alpha = 0 included.
* The backward's chunk form: the reverse mode of the chunk form above,
  chained over chunks through dL/dS, against the oracle's backward.
"""
import numpy as np
import pytest

import gdn2_inputs as gi
import oracle

NAMES = ("q", "k", "v", "alpha", "b", "w")


def f64(inp):
    return {n: inp[n].double().numpy() for n in NAMES}


def chunk_forward(q, k, v, al, b, w, S, C, pairwise=False):
    """One sequence and head: q, k, b, al [T, dk]; v, w [T, dv]; S [dk, dv].
    Returns (o [T, dv], S_final, per-chunk caches for the backward)."""
    T = q.shape[0]
    o = np.zeros((T, v.shape[1]))
    caches = []
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        qc, kc, vc, ac, bc, wc = q[sl], k[sl], v[sl], al[sl], b[sl], w[sl]
        n = qc.shape[0]
        with np.errstate(divide="ignore"):
            lg = np.log(ac)
        F = decay_pairs(lg, ac, pairwise)                  # F[t, s, c] = e^{g_t - g_s}, s <= t
        g = np.cumsum(lg, axis=0)
        gam = np.exp(g)                                    # e^{g_t}
        gC = gam[-1]
        # e^{g_C - g_s} as the suffix product of the alphas after s
        tail = np.ones_like(ac)
        for s in range(n - 2, -1, -1):
            tail[s] = tail[s + 1] * ac[s + 1]
        e = bc * kc
        A = np.einsum("tc,sc,tsc->ts", e, kc, F) * np.tri(n, k=-1)
        P = np.einsum("tc,sc,tsc->ts", qc, kc, F) * np.tri(n)
        Tm = np.linalg.inv(np.eye(n) + A)
        U = wc * vc
        ES = e * gam
        Y = U - ES @ S
        Z = Tm @ Y
        O = (qc * gam) @ S + P @ Z
        KB = kc * tail
        S_new = gC[:, None] * S + KB.T @ Z
        o[sl] = O
        caches.append(dict(sl=sl, q=qc, k=kc, e=e, b=bc, w=wc, v=vc, al=ac, F=F, gam=gam, gC=gC, tail=tail,
                           A=A, P=P, T=Tm, Y=Y, Z=Z, KB=KB, S=S.copy()))
        S = S_new
    return o, S, caches


def decay_pairs(lg, ac, pairwise):
    """F[t, s, c] = e^{g_t - g_s} for s <= t (zero above), per channel.
    pairwise=False: the plain difference of cumulative sums (no alpha = 0).
    pairwise=True: the kernels' factorisation per 16-token sub-block, every
    factor a sum of log decays, the diagonal blocks of sub-blocks decaying
    by more than 2^-64 as running products of the alphas."""
    n, d = lg.shape
    F = np.zeros((n, n, d))
    if not pairwise:
        g = np.cumsum(lg, axis=0)
        for t in range(n):
            F[t, :t + 1] = np.exp(g[t] - g[:t + 1])
        return F
    nb = -(-n // 16)
    tot = np.array([lg[16 * I:16 * I + 16].sum(axis=0) for I in range(nb)])    # sub-block log decays
    for t in range(n):
        I = t // 16
        row = lg[16 * I:t + 1].sum(axis=0)                                       # g_t - rho_I
        for s in range(t + 1):
            J = s // 16
            if J < I:
                key = lg[s + 1:16 * J + 16].sum(axis=0)                          # rho_{J+1} - g_s
                mid = tot[J + 1:I].sum(axis=0)                                   # rho_I - rho_{J+1}
                F[t, s] = np.exp(row) * np.exp(key) * np.exp(mid)
            elif np.all(tot[I] >= -64 * np.log(2.0)):
                F[t, s] = np.exp(row) * np.exp(-lg[16 * I:s + 1].sum(axis=0))    # e^{rho_I - g_s} bounded
            else:
                F[t, s] = np.prod(ac[s + 1:t + 1], axis=0)                       # running product
    return F


def run_chunked(inp, C, pairwise=False):
    x = f64(inp)
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    S0 = inp["S0"].double().numpy() if inp.get("S0") is not None else np.zeros((B, H, dk, dv))
    o = np.zeros((B, T, H, dv))
    Sf = np.zeros((B, H, dk, dv))
    for bb in range(B):
        for hh in range(H):
            args = [x[n][bb, :, hh] for n in NAMES]
            o[bb, :, hh], Sf[bb, hh], _ = chunk_forward(*args, S0[bb, hh].copy(), C, pairwise)
    return o, Sf


def rel(x, ref):
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


@pytest.mark.parametrize("C", [8, 10, 16, 64])
def test_chunk_form_equals_token_recurrence(C):
    inp = gi.make_chunk_inputs(2, 150, 2, 16, 16, "f32", seed=5, s0="normal")
    o, Sf = run_chunked(inp, C)
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    assert rel(o, o_ref) < 1e-12 and rel(Sf, S_ref) < 1e-12


@pytest.mark.parametrize("kind", ["strong", "spiky", "zero"])
def test_kernel_factorisation_with_extreme_decay(kind):
    """The kernels' per-sub-block factorisation (sums of log decays only;
    pairwise diagonal blocks past 2^-64) equals the oracle with decays of
    1e-6, zeros, and everything zero."""
    if kind == "zero":
        inp = gi.make_chunk_inputs(1, 100, 2, 16, 16, "f32", seed=6, s0="normal")
        inp["alpha"] = inp["alpha"] * 0
    else:
        par = (dict(logit_mean=-2.0, logit_std=2.0, tiny_frac=0.02, tiny=1e-6, zero_frac=0.02) if kind == "strong"
               else dict(logit_mean=3.0, logit_std=1.0, tiny_frac=0.01, tiny=1e-6, zero_frac=0.01))
        inp = gi.make_strong_decay_inputs(1, 100, 2, 16, 16, "f32", seed=7, s0="normal", **par)
    o, Sf = run_chunked(inp, 64, pairwise=True)
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    assert np.isfinite(o).all() and np.isfinite(Sf).all()
    assert rel(o, o_ref) < 1e-12 and rel(Sf, S_ref) < 1e-12


def test_plain_factorisation_fails_where_the_kernels_switch():
    """Pin of the switch itself: with alpha = 0 in a sub-block the plain
    difference of cumulative sums gives NaN, which is why the kernels form
    every factor as a sum and the diagonal blocks pairwise."""
    inp = gi.make_chunk_inputs(1, 40, 1, 16, 16, "f32", seed=8, s0="normal")
    inp["alpha"][0, 5, 0, 3] = 0.0
    with np.errstate(invalid="ignore"):
        o, _ = run_chunked(inp, 16, pairwise=False)
    assert np.isnan(o).any()
    o, _ = run_chunked(inp, 16, pairwise=True)
    assert np.isfinite(o).all()


def chunk_backward(caches, dO_all, dH):
    """Reverse mode of chunk_forward for one sequence and head, from the
    last chunk, given dL/do and dL/dS_final.  Returns the input gradients
    and dL/dS0.  Per chunk (the backward kernels' formulas):
      dZ = P^T dO + KB dH,  dY = T^T dZ,  dA = -strict_lower(dY Z^T),
      dP = lower(dO Z^T),  dS = Diag(gamma_C) dH + (q e^g)^T dO - (e e^g)^T dY,
    then the chain rule through e^{g_t - g_s}, e^{g_t}, e^{g_C - g_t} to
    q, k, b, alpha, and dv = dY (.) w, dw = dY (.) v."""
    out = {n: [] for n in ("dq", "dk", "dv", "dalpha", "db", "dw")}
    for cc in reversed(caches):
        dO = dO_all[cc["sl"]]
        S, P, Tm, Z, KB, F = cc["S"], cc["P"], cc["T"], cc["Z"], cc["KB"], cc["F"]
        q, k, e, gam, tail, gC = cc["q"], cc["k"], cc["e"], cc["gam"], cc["tail"], cc["gC"]
        n = q.shape[0]
        dZ = P.T @ dO + KB @ dH
        dY = Tm.T @ dZ
        dA = -(dY @ Z.T) * np.tri(n, k=-1)
        dP = (dO @ Z.T) * np.tri(n)
        dQS = dO @ S.T                                     # d(q e^g)
        dES = -(dY @ S.T)                                  # d(e e^g)
        dKB = Z @ dH.T                                     # d(k e^{g_C - g})
        dgam = np.sum(dH * S, axis=1)                      # d(gamma_C)
        dS = gC[:, None] * dH + (q * gam).T @ dO - (e * gam).T @ dY
        dq = dQS * gam + np.einsum("ts,sc,tsc->tc", dP, k, F)
        de = dES * gam + np.einsum("ts,sc,tsc->tc", dA, k, F)
        dkk = dKB * tail + np.einsum("ts,tc,tsc->sc", dP, q, F) + np.einsum("ts,tc,tsc->sc", dA, e, F)
        # d g_t: +(row side) for e^{g_t}, e^{g_t - g_s}; -(key side) for e^{-g_s}
        dg = q * dQS * gam + e * dES * gam
        dg += np.einsum("ts,tc,sc,tsc->tc", dP, q, k, F) + np.einsum("ts,tc,sc,tsc->tc", dA, e, k, F)
        dg -= np.einsum("ts,tc,sc,tsc->sc", dP, q, k, F) + np.einsum("ts,tc,sc,tsc->sc", dA, e, k, F)
        dg -= k * dKB * tail
        dgC = gC * dgam + np.sum(k * dKB * tail, axis=0)   # d g_C
        dlog = np.cumsum(dg[::-1], axis=0)[::-1] + dgC     # d ln(alpha_s) = sum_{t >= s} dg_t + d g_C
        out["dq"].append(dq)
        out["dk"].append(dkk + cc["b"] * de)
        out["db"].append(k * de)
        out["dv"].append(dY * cc["w"])
        out["dw"].append(dY * cc["v"])
        out["dalpha"].append(dlog / cc["al"])
        dH = dS
    return {n: np.concatenate(x[::-1], axis=0) for n, x in out.items()}, dH


@pytest.mark.parametrize("C", [16, 64])
def test_chunk_backward_equals_oracle_backward(C):
    inp = gi.make_chunk_inputs(1, 150, 2, 16, 16, "f32", seed=9, s0="normal")
    grads = gi.make_bwd_grads(1, 150, 2, 16, 16, "f32", seed=9)
    x = f64(inp)
    dO = grads["dout"].double().numpy()
    dSf = grads["dS_final"].double().numpy()
    ref = oracle.bwd(*(inp[n] for n in NAMES), grads["dout"], S0=inp["S0"], dS_final=grads["dS_final"])
    for hh in range(2):
        args = [x[n][0, :, hh] for n in NAMES]
        _, _, caches = chunk_forward(*args, inp["S0"][0, hh].double().numpy(), C)
        got, dS0 = chunk_backward(caches, dO[0, :, hh], dSf[0, hh])
        for name in got:
            assert rel(got[name], ref[name][0, :, hh]) < 1e-10, name
        assert rel(dS0, ref["dS0"][0, hh]) < 1e-10


def chunk_forward_r1(q, k, v, al, b, w, S, C):
    """Chunk form of reading R1 (erase along b (.) k, read with k) for one
    sequence and head.  With R = [r_t] the reads D_t^T k_t of the chunk:
      (I + A') R = Kchk S0 + B' U,  A' = strict_lower(Kchk Ehat^T),
      B' = strict_lower(Kchk Khat^T),  R = W' S0 + Ut',  W' = T' Kchk,
      Ut' = T' B' U,  T' = (I + A')^-1,
      O = (Qchk - P_e W') S0 + (P_k U - P_e Ut'),  P_e = lower(Qchk Ehat^T),
      P_k = lower(Qchk Khat^T),
      S_C = Diag(gamma_C) S0 + Kbar^T U - Ebar^T R
    (Kchk = k e^g, Ehat = e e^-g, Khat = k e^-g, Qchk = q e^g, Kbar =
    k e^{g_C - g}, Ebar = e e^{g_C - g})."""
    T = q.shape[0]
    o = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        qc, kc, vc, ac, bc, wc = q[sl], k[sl], v[sl], al[sl], b[sl], w[sl]
        n = qc.shape[0]
        g = np.cumsum(np.log(ac), axis=0)
        gam, gC = np.exp(g), np.exp(g[-1])
        e = bc * kc
        U = wc * vc
        Kc, Eh, Kh, Qc = kc * gam, e / gam, kc / gam, qc * gam
        Ap = (Kc @ Eh.T) * np.tri(n, k=-1)
        Bp = (Kc @ Kh.T) * np.tri(n, k=-1)
        Pe = (Qc @ Eh.T) * np.tri(n)
        Pk = (Qc @ Kh.T) * np.tri(n)
        Tp = np.linalg.inv(np.eye(n) + Ap)
        Wp = Tp @ Kc
        Utp = Tp @ (Bp @ U)
        o[sl] = (Qc - Pe @ Wp) @ S + (Pk @ U - Pe @ Utp)
        R = Wp @ S + Utp
        S = gC[:, None] * S + (kc * gC / gam).T @ U - (e * gC / gam).T @ R
    return o, S


@pytest.mark.parametrize("C", [8, 16, 64])
def test_r1_chunk_form_equals_token_recurrence(C):
    inp = gi.make_chunk_inputs(1, 150, 2, 16, 16, "f32", seed=11, s0="normal")
    x = f64(inp)
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"], rule="R1")
    for hh in range(2):
        o, S = chunk_forward_r1(*(x[n][0, :, hh] for n in NAMES), inp["S0"][0, hh].double().numpy(), C)
        assert rel(o, o_ref[0, :, hh]) < 1e-12 and rel(S, S_ref[0, hh]) < 1e-12
