"""Pins of the oracle's backward (``oracle.bwd``, the hand-derived reverse-mode
derivative of the token recurrence).  Each test fixes it against something
other than itself: central finite differences of the forward oracle, float64
autograd of an independent PyTorch transcription of the forward, and the
linearity of a gradient in the incoming gradients.  CPU only."""
import numpy as np
import pytest
import torch

import oracle

NAMES = ("q", "k", "v", "alpha", "b", "w")


def rand_inputs(rng, B, T, H, dk, dv):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    return {
        "q": q, "k": k, "v": rng.standard_normal((B, T, H, dv)),
        "alpha": 1.0 / (1.0 + np.exp(-rng.normal(2.0, 1.0, (B, T, H, dk)))),
        "b": 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, dk)))),
        "w": 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H, dv)))),
    }


def loss(x, S0, do, dSf, cu=None):
    """L = <do, o> + <dSf, S_final>, so dL/do = do and dL/dS_final = dSf."""
    o, Sf = oracle.fwd(*(x[n] for n in NAMES), S0=S0, cu_seqlens=cu)
    return float(np.sum(do * o) + np.sum(dSf * Sf))


def test_bwd_matches_finite_differences():
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 2, 5, 1, 3, 4
    x = rand_inputs(rng, B, T, H, dk, dv)
    S0 = rng.normal(0.0, 0.3, (B, H, dk, dv))
    do = rng.standard_normal((B, T, H, dv))
    dSf = rng.standard_normal((B, H, dk, dv))
    g = oracle.bwd(*(x[n] for n in NAMES), do, S0=S0, dS_final=dSf)
    h = 1e-6
    targets = [(n, x[n], "d" + n) for n in NAMES] + [("S0", S0, "dS0")]
    for name, arr, gname in targets:
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + h
            lp = loss(x, S0, do, dSf)
            arr[idx] = keep - h
            lm = loss(x, S0, do, dSf)
            arr[idx] = keep
            fd[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - g[gname])) / np.max(np.abs(fd))
        assert err < 1e-7, (name, err)


def torch_forward(x, S0, cu):
    """Independent float64 transcription of the recurrence for autograd:
    decay rows of S, read with b (.) k, delta value w (.) v - read, write
    along k, read out after the update."""
    B, T, H, dk = x["q"].shape
    dv = x["v"].shape[-1]
    seqs = [(0, int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)] if cu is not None \
        else [(n, 0, T) for n in range(B)]
    outs = torch.zeros(B, T, H, dv, dtype=torch.float64)
    finals = []
    for si, (n, a, e) in enumerate(seqs):
        fin_h = []
        for h in range(H):
            S = S0[si, h]
            for t in range(a, e):
                q, k, v = x["q"][n, t, h], x["k"][n, t, h], x["v"][n, t, h]
                al, b, w = x["alpha"][n, t, h], x["b"][n, t, h], x["w"][n, t, h]
                D = al[:, None] * S
                z = w * v - D.t() @ (b * k)
                S = D + torch.outer(k, z)
                outs = outs.index_put((torch.tensor(n), torch.tensor(t), torch.tensor(h)), S.t() @ q)
            fin_h.append(S)
        finals.append(torch.stack(fin_h))
    return outs, torch.stack(finals)


@pytest.mark.parametrize("varlen", [False, True])
def test_bwd_matches_autograd_across_checkpoint_segments(varlen):
    rng = np.random.default_rng(12 + varlen)
    if varlen:  # two sequences, one spanning two of the oracle's 64-token segments
        B, T, cu = 1, 150, np.array([0, 70, 150], dtype=np.int32)
        N = 2
    else:
        B, T, cu = 2, 140, None
        N = B
    H, dk, dv = 2, 5, 6
    x = rand_inputs(rng, B, T, H, dk, dv)
    S0 = rng.normal(0.0, 0.3, (N, H, dk, dv))
    do = rng.standard_normal((B, T, H, dv))
    dSf = rng.standard_normal((N, H, dk, dv))
    g = oracle.bwd(*(x[n] for n in NAMES), do, S0=S0, dS_final=dSf, cu_seqlens=cu)
    xt = {n: torch.tensor(x[n], requires_grad=True) for n in NAMES}
    S0t = torch.tensor(S0, requires_grad=True)
    o, Sf = torch_forward(xt, S0t, cu)
    L = (o * torch.tensor(do)).sum() + (Sf * torch.tensor(dSf)).sum()
    L.backward()
    for n in NAMES:
        ref = xt[n].grad.numpy()
        err = np.max(np.abs(g["d" + n] - ref)) / np.max(np.abs(ref))
        assert err < 1e-11, (n, err)
    ref = S0t.grad.numpy()
    assert np.max(np.abs(g["dS0"] - ref)) / np.max(np.abs(ref)) < 1e-11


def test_bwd_is_linear_in_incoming_gradients():
    rng = np.random.default_rng(13)
    B, T, H, dk, dv = 1, 40, 1, 4, 3
    x = rand_inputs(rng, B, T, H, dk, dv)
    do1, do2 = rng.standard_normal((2, B, T, H, dv))
    dS1, dS2 = rng.standard_normal((2, B, H, dk, dv))
    g1 = oracle.bwd(*(x[n] for n in NAMES), do1, dS_final=dS1)
    g2 = oracle.bwd(*(x[n] for n in NAMES), do2, dS_final=dS2)
    g12 = oracle.bwd(*(x[n] for n in NAMES), 2 * do1 - 3 * do2, dS_final=2 * dS1 - 3 * dS2)
    for key in g1:
        ref = 2 * g1[key] - 3 * g2[key]
        assert np.max(np.abs(g12[key] - ref)) <= 1e-12 * max(np.max(np.abs(ref)), 1.0), key


def test_bwd_zero_incoming_gradient_gives_zero():
    rng = np.random.default_rng(14)
    x = rand_inputs(rng, 1, 9, 2, 3, 3)
    g = oracle.bwd(*(x[n] for n in NAMES), np.zeros((1, 9, 2, 3)))
    for key, val in g.items():
        assert np.all(val == 0.0), key


def test_layer_prep_bwd_matches_finite_differences():
    """The chain rule of oracle/layer_prep.py against central differences of
    the loss through layer_prep and the forward oracle, for per-channel and
    per-(token, head) gate layouts."""
    from oracle import layer_prep as lp
    rng = np.random.default_rng(15)
    B, T, H, dk, dv = 1, 6, 1, 3, 2
    for scalar in (False, True):
        gshape = (B, T, H) if scalar else None
        raw = {
            "q": rng.standard_normal((B, T, H, dk)) * 2.0,
            "k": rng.standard_normal((B, T, H, dk)) * 0.7,
            "v": rng.standard_normal((B, T, H, dv)),
            "alpha": np.log(1.0 / (1.0 + np.exp(-rng.normal(2.0, 1.0, gshape or (B, T, H, dk))))),
            "b": rng.standard_normal(gshape or (B, T, H, dk)),
            "w": rng.standard_normal(gshape or (B, T, H, dv)),
        }
        raw["q"][0, 2, 0] = 0.0  # a zero row stays zero, and so does its gradient
        S0 = rng.normal(0.0, 0.3, (B, H, dk, dv))
        do = rng.standard_normal((B, T, H, dv))
        dSf = rng.standard_normal((B, H, dk, dv))

        def prepared(r):
            p = lp.layer_prep(r["q"], r["k"], r["alpha"], r["b"], r["w"])
            full = {x: (p[x][..., None] * np.ones(dk if x in ("alpha", "b") else dv) if p[x].ndim == 3 else p[x])
                    for x in ("q", "k", "alpha", "b", "w")}
            full["v"] = r["v"]
            return full

        def L(r):
            p = prepared(r)
            o, Sf = oracle.fwd(*(p[n] for n in NAMES), S0=S0)
            return float(np.sum(do * o) + np.sum(dSf * Sf))

        p = prepared(raw)
        gp = oracle.bwd(*(p[n] for n in NAMES), do, S0=S0, dS_final=dSf)
        g = lp.layer_prep_bwd(raw["q"], raw["k"], raw["alpha"], raw["b"], raw["w"], gp)
        h = 1e-6
        for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("alpha", "dalpha"), ("b", "db"), ("w", "dw")):
            arr = raw[name]
            fd = np.zeros_like(arr)
            skip = np.zeros(arr.shape, dtype=bool)
            if name == "q":  # normalisation is not differentiable at the zero row
                skip[0, 2, 0] = True
            for idx in np.ndindex(arr.shape):
                if skip[idx]:
                    continue
                keep = arr[idx]
                arr[idx] = keep + h
                lp_ = L(raw)
                arr[idx] = keep - h
                lm = L(raw)
                arr[idx] = keep
                fd[idx] = (lp_ - lm) / (2 * h)
            assert g[gname].shape == arr.shape, name
            err = np.max(np.abs(np.where(skip, 0.0, fd - g[gname]))) / np.max(np.abs(fd))
            assert err < 1e-7, (scalar, name, err)
        assert np.all(g["dq"][0, 2, 0] == 0.0)


def test_per_token_gate_gradients_are_channel_sums():
    """Gates given per (token, head) and broadcast over the channels: their
    gradient (oracle.bwd per channel, summed by sum_to_layout) against
    central differences of the loss in the compact gate."""
    from oracle import layer_prep as lp
    rng = np.random.default_rng(16)
    B, T, H, dk, dv = 1, 7, 2, 3, 4
    x = rand_inputs(rng, B, T, H, dk, dv)
    compact = {"b": rng.uniform(0.1, 0.9, (B, T, H)), "w": rng.uniform(0.1, 0.9, (B, T, H)),
               "alpha": rng.uniform(0.5, 0.99, (B, T, H))}
    do = rng.standard_normal((B, T, H, dv))

    def full(c):
        f = dict(x)
        f["b"] = np.repeat(c["b"][..., None], dk, -1)
        f["w"] = np.repeat(c["w"][..., None], dv, -1)
        f["alpha"] = np.repeat(c["alpha"][..., None], dk, -1)
        return f

    f = full(compact)
    gfull = oracle.bwd(*(f[n] for n in NAMES), do)
    h = 1e-6
    for name in ("b", "w", "alpha"):
        got = lp.sum_to_layout(gfull["d" + name], compact[name])
        assert got.shape == compact[name].shape
        fd = np.zeros_like(compact[name])
        for idx in np.ndindex(fd.shape):
            keep = compact[name][idx]
            compact[name][idx] = keep + h
            fp = full(compact)
            lpl = float(np.sum(do * oracle.fwd(*(fp[n] for n in NAMES))[0]))
            compact[name][idx] = keep - h
            fm = full(compact)
            lmi = float(np.sum(do * oracle.fwd(*(fm[n] for n in NAMES))[0]))
            compact[name][idx] = keep
            fd[idx] = (lpl - lmi) / (2 * h)
        assert np.max(np.abs(fd - got)) / np.max(np.abs(fd)) < 1e-7, name
