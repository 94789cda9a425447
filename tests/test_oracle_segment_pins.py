"""Pins of the oracle's segment map (``oracle.segment_map``: S_out = Phi S_in
+ Psi over a run of tokens) and of the exclusive scan that chains such maps
(``oracle.segment_combine``).  Each is fixed against something other than
itself: the C token-by-token forward run from arbitrary states, the closed
form when nothing is erased, the explicit matrix of a single token, and the
composition of two halves.  CPU only."""
import numpy as np

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


def rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


def test_map_reproduces_the_forward_from_any_state():
    rng = np.random.default_rng(21)
    for cu in (None, np.array([0, 13, 13, 40, 71], dtype=np.int32)):
        B, T = (3, 37) if cu is None else (1, 71)
        H, dk, dv = 2, 5, 4
        x = rand_inputs(rng, B, T, H, dk, dv)
        Phi, Psi = oracle.segment_map(*(x[n] for n in NAMES), cu_seqlens=cu)
        N = Phi.shape[0]
        for _ in range(2):
            S = rng.standard_normal((N, H, dk, dv))
            _, Sf = oracle.fwd(*(x[n] for n in NAMES), S0=S, cu_seqlens=cu)
            assert rel(Phi @ S + Psi, Sf) < 1e-12
        if cu is not None:  # the empty sequence maps every state to itself
            assert np.array_equal(Phi[1], np.broadcast_to(np.eye(dk), (H, dk, dk)))
            assert np.all(Psi[1] == 0.0)


def test_single_token_map_is_the_explicit_matrix():
    rng = np.random.default_rng(22)
    x = rand_inputs(rng, 1, 1, 1, 6, 3)
    k, b, al = x["k"][0, 0, 0], x["b"][0, 0, 0], x["alpha"][0, 0, 0]
    A = (np.eye(6) - np.outer(k, b * k)) @ np.diag(al)
    Phi, Psi = oracle.segment_map(*(x[n] for n in NAMES))
    assert rel(Phi[0, 0], A) < 1e-14
    assert rel(Psi[0, 0], np.outer(k, x["w"][0, 0, 0] * x["v"][0, 0, 0])) < 1e-14


def test_without_erase_the_map_is_the_decay_product():
    # b = 0: nothing is read back, S' = Diag(alpha) S + k (w (.) v)^T
    rng = np.random.default_rng(23)
    T, dk, dv = 9, 4, 3
    x = rand_inputs(rng, 1, T, 1, dk, dv)
    x["b"][:] = 0.0
    Phi, Psi = oracle.segment_map(*(x[n] for n in NAMES))
    al, k, wv = x["alpha"][0, :, 0], x["k"][0, :, 0], x["w"][0, :, 0] * x["v"][0, :, 0]
    assert rel(Phi[0, 0], np.diag(np.prod(al, axis=0))) < 1e-14
    ref = sum(np.prod(al[t + 1:], axis=0)[:, None] * np.outer(k[t], wv[t]) for t in range(T))
    assert rel(Psi[0, 0], ref) < 1e-13


def test_maps_of_two_halves_compose():
    rng = np.random.default_rng(24)
    T, H, dk, dv, m = 30, 2, 4, 5, 11
    x = rand_inputs(rng, 1, T, H, dk, dv)
    whole = oracle.segment_map(*(x[n] for n in NAMES))
    halves = oracle.segment_map(*(x[n] for n in NAMES), cu_seqlens=np.array([0, m, T], dtype=np.int32))
    (P1, P2), (Q1, Q2) = halves
    assert rel(whole[0][0], P2 @ P1) < 1e-12
    assert rel(whole[1][0], P2 @ Q1 + Q2) < 1e-12


def test_combine_then_segments_reproduce_the_sequence():
    rng = np.random.default_rng(25)
    T, H, dk, dv = 100, 2, 4, 3
    x = rand_inputs(rng, 1, T, H, dk, dv)
    S0 = rng.normal(0.0, 0.3, (1, H, dk, dv))
    cu = np.array([0, 17, 50, 50, 64, 100], dtype=np.int32)   # five segments, one empty
    Phi, Psi = oracle.segment_map(*(x[n] for n in NAMES), cu_seqlens=cu)
    S_in, S_fin = oracle.segment_combine(Phi, Psi, S0[0])
    o_seg, Sf_seg = oracle.fwd(*(x[n] for n in NAMES), S0=S_in, cu_seqlens=cu)
    o, Sf = oracle.fwd(*(x[n] for n in NAMES), S0=S0)
    assert rel(o_seg, o) < 1e-12
    assert rel(S_fin, Sf[0]) < 1e-12
    assert rel(Sf_seg[-1], Sf[0]) < 1e-12
    assert np.array_equal(S_in[0], S0[0])
    assert np.array_equal(S_in[3], S_in[2])   # the empty segment passes its state on


def test_combine_without_segments_returns_the_initial_state():
    S0 = np.arange(12.0).reshape(1, 3, 4)
    S_in, Sf = oracle.segment_combine(np.zeros((0, 1, 3, 3)), np.zeros((0, 1, 3, 4)), S0)
    assert S_in.shape == (0, 1, 3, 4)
    assert np.array_equal(Sf, S0)
