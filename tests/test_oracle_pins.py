"""Pins of the CPU oracle: each test fixes part of the oracle against
something other than the oracle itself (a hand-worked example, a textbook
recurrence, a closed form, an invariant).  CPU only."""
from fractions import Fraction
import os

import numpy as np
import pytest
import torch

import gdn2_inputs as gi
import oracle
from oracle import pins, reference_np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _head(x):
    """[T, d] float64 -> [1, T, 1, d]"""
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64)[None, :, None, :])


def run_head(q, k, v, alpha, b, w, S0=None, rule="R5"):
    o, Sf = oracle.fwd(_head(q), _head(k), _head(v), _head(alpha), _head(b), _head(w),
                       None if S0 is None else np.asarray(S0, dtype=np.float64)[None, None],
                       rule=rule)
    return o[0, :, 0], Sf[0, 0]


def rand_head(rng, T, dk, dv, unit_k=True):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    if unit_k:
        q /= np.linalg.norm(q, axis=1, keepdims=True)
        k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    alpha = 1.0 / (1.0 + np.exp(-rng.normal(3.0, 1.0, (T, dk))))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, dk))))
    w = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, dv))))
    S0 = rng.normal(0.0, 0.1, (dk, dv))
    return q, k, v, alpha, b, w, S0


def rel(a, ref):
    return float(np.max(np.abs(a - ref)) / max(np.max(np.abs(ref)), 1e-300))


# ---------------------------------------------------------------- golden --
def _parse_golden():
    vals = {}
    with open(os.path.join(GOLDEN, "worked_example_2x2.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rhs = line.split(":", 1)
            rows = [[float(Fraction(x)) for x in part.split()] for part in rhs.split(";")]
            vals[key.strip()] = np.array(rows, dtype=np.float64)
    return vals


@pytest.mark.parametrize("rule", ["R5", "R1"])
def test_hand_worked_example(rule):
    g = _parse_golden()
    S0 = g["S0"].reshape(2, 2)
    o, Sf = run_head(g["q"], g["k"], g["v"], g["alpha"], g["b"], g["w"], S0, rule=rule)
    # dyadic rationals: exact in float64
    np.testing.assert_array_equal(o, g[f"{rule}.o"])
    np.testing.assert_array_equal(Sf, g[f"{rule}.S_final"].reshape(2, 2))


# ------------------------------------------------------- reductions (P1) --
@pytest.mark.parametrize("dk,dv,T", [(16, 16, 64), (64, 32, 96)])
def test_P1a_reduces_to_kda(dk, dv, T):
    rng = np.random.default_rng(11)
    q, k, v, alpha, _, _, S0 = rand_head(rng, T, dk, dv)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    b = np.repeat(beta[:, None], dk, axis=1)
    w = np.repeat(beta[:, None], dv, axis=1)
    o, Sf = run_head(q, k, v, alpha, b, w, S0)
    o_ref, S_ref = pins.kda_textbook(q, k, v, alpha, beta, S0)
    assert rel(o, o_ref) < 1e-12
    assert rel(Sf, S_ref) < 1e-12


def test_P1b_reduces_to_gated_deltanet():
    rng = np.random.default_rng(12)
    T, dk, dv = 80, 16, 24
    q, k, v, _, _, _, S0 = rand_head(rng, T, dk, dv)
    a = 1.0 / (1.0 + np.exp(-rng.normal(3.0, 1.0, T)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    alpha = np.repeat(a[:, None], dk, axis=1)
    o, Sf = run_head(q, k, v, alpha, np.repeat(beta[:, None], dk, 1),
                     np.repeat(beta[:, None], dv, 1), S0)
    o_ref, S_ref = pins.gdn_textbook(q, k, v, a, beta, S0)
    assert rel(o, o_ref) < 1e-12
    assert rel(Sf, S_ref) < 1e-12


def test_P1c_reduces_to_deltanet():
    rng = np.random.default_rng(13)
    T, dk, dv = 80, 16, 16
    q, k, v, _, _, _, S0 = rand_head(rng, T, dk, dv)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    o, Sf = run_head(q, k, v, np.ones((T, dk)), np.repeat(beta[:, None], dk, 1),
                     np.repeat(beta[:, None], dv, 1), S0)
    o_ref, S_ref = pins.deltanet_textbook(q, k, v, beta, S0)
    assert rel(o, o_ref) < 1e-12
    assert rel(Sf, S_ref) < 1e-12


# ------------------------------------------------------ closed forms (P2) --
def test_P2_linear_attention_closed_form():
    rng = np.random.default_rng(21)
    T, dk, dv = 48, 16, 8
    q, k, v, _, _, _, S0 = rand_head(rng, T, dk, dv, unit_k=False)
    o, _ = run_head(q, k, v, np.ones((T, dk)), np.zeros((T, dk)), np.ones((T, dv)), S0)
    assert rel(o, pins.linear_attention_closed(q, k, v, S0)) < 1e-12


def test_P2prime_channel_decay_closed_form():
    rng = np.random.default_rng(22)
    T, dk, dv = 40, 8, 8
    q, k, v, alpha, _, _, S0 = rand_head(rng, T, dk, dv)
    o, _ = run_head(q, k, v, alpha, np.zeros((T, dk)), np.ones((T, dv)), S0)
    assert rel(o, pins.decayed_linear_closed(q, k, v, alpha, S0)) < 1e-12


# ------------------------------------------------------------ invariants --
def test_P3_orthonormal_exact_recall():
    rng = np.random.default_rng(31)
    dk, dv, T = 32, 16, 32
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:, :T].T.copy()
    v = rng.standard_normal((T, dv))
    q = rng.standard_normal((T, dk))
    _, Sf = run_head(q, k, v, np.ones((T, dk)), np.ones((T, dk)), np.ones((T, dv)))
    np.testing.assert_allclose(Sf.T @ k.T, v.T, atol=1e-12)


def test_P4_self_read_returns_written_value():
    """b = 1, unit keys, q = k: the read-out equals the gated value w (.) v."""
    rng = np.random.default_rng(41)
    T, dk, dv = 64, 16, 12
    q, k, v, alpha, _, w, S0 = rand_head(rng, T, dk, dv)
    o, _ = run_head(k, k, v, alpha, np.ones((T, dk)), w, S0)
    np.testing.assert_allclose(o, w * v, atol=1e-12)


def test_P5_pure_decay():
    rng = np.random.default_rng(51)
    T, dk, dv = 30, 8, 8
    q, k, v, alpha, _, _, S0 = rand_head(rng, T, dk, dv)
    _, Sf = run_head(q, k, v, alpha, np.zeros((T, dk)), np.zeros((T, dv)), S0)
    np.testing.assert_allclose(Sf, np.prod(alpha, axis=0)[:, None] * S0, rtol=1e-13, atol=0)


def test_P6_erase_gate_two_is_a_reflection():
    """b = 2, alpha = 1, w = 0, unit k: each step is a Householder reflection,
    so the Frobenius norm of the state is preserved (the b in [0,2] range of
    the aixai.ru ablation section; no clamping)."""
    rng = np.random.default_rng(61)
    dk, dv = 16, 8
    q, k, v, _, _, _, S0 = rand_head(rng, 20, dk, dv)
    S = S0[None, None].copy()
    n0 = np.linalg.norm(S0)
    for t in range(20):
        one = lambda x: x[t][None, None]
        _, S = oracle.decode(one(q), one(k), one(v), np.ones((1, 1, dk)), 2 * np.ones((1, 1, dk)),
                             np.zeros((1, 1, dv)), S)
        assert abs(np.linalg.norm(S) - n0) < 1e-12 * n0
    assert np.max(np.abs(S[0, 0] - S0)) > 1e-3  # it did move


# --------------------------------------------------- structure (P7 - P9) --
def test_P7_split_resume_and_varlen():
    inp = gi.make_chunk_inputs(2, 100, 3, 16, 12, "f32", seed=71, s0="normal")
    args = [inp[x] for x in ("q", "k", "v", "alpha", "b", "w")]
    o, Sf = oracle.fwd(*args, S0=inp["S0"])
    T1 = 37
    o1, S1 = oracle.fwd(*[a[:, :T1] for a in args], S0=inp["S0"])
    o2, S2 = oracle.fwd(*[a[:, T1:] for a in args], S0=S1)
    np.testing.assert_array_equal(np.concatenate([o1, o2], axis=1), o)
    np.testing.assert_array_equal(S2, Sf)
    # packed: the two batch rows laid end to end are two sequences
    packed = [a.reshape(1, 200, 3, -1) for a in args]
    cu = np.array([0, 100, 200], dtype=np.int32)
    op, Sp = oracle.fwd(*packed, S0=inp["S0"], cu_seqlens=cu)
    np.testing.assert_array_equal(op.reshape(o.shape), o)
    np.testing.assert_array_equal(Sp, Sf)


def test_P8_linear_in_state_and_values():
    inp = gi.make_chunk_inputs(1, 50, 2, 8, 8, "f32", seed=81, s0="normal")
    q, k, v, alpha, b, w = (inp[x] for x in ("q", "k", "v", "alpha", "b", "w"))
    rng = np.random.default_rng(82)
    v2 = rng.standard_normal(v.shape)
    S2 = rng.standard_normal(inp["S0"].shape)
    c1, c2 = 0.75, -1.5
    oa, Sa = oracle.fwd(q, k, v, alpha, b, w, S0=inp["S0"])
    ob, Sb = oracle.fwd(q, k, v2, alpha, b, w, S0=S2)
    oc, Sc = oracle.fwd(q, k, c1 * v.double().numpy() + c2 * v2, alpha, b, w,
                        S0=c1 * inp["S0"].double().numpy() + c2 * S2)
    assert rel(oc, c1 * oa + c2 * ob) < 1e-12
    assert rel(Sc, c1 * Sa + c2 * Sb) < 1e-12


def test_P9_decode_steps_equal_forward():
    d = gi.make_decode_inputs(3, 2, 16, 8, "f32", seed=91, steps=12)
    S = d["S"].double().numpy()
    outs = []
    for t in range(12):
        o, S = oracle.decode(*(d[x][t] for x in ("q", "k", "v", "alpha", "b", "w")), S)
        outs.append(o)
    seq = {x: d[x].permute(1, 0, 2, 3).contiguous() for x in ("q", "k", "v", "alpha", "b", "w")}
    of, Sf = oracle.fwd(*(seq[x] for x in ("q", "k", "v", "alpha", "b", "w")), S0=d["S"])
    np.testing.assert_array_equal(np.stack(outs, axis=1), of)
    np.testing.assert_array_equal(S, Sf)


def test_c_oracle_matches_numpy_transcription_small_workloads():
    for name in ("tiny_1x64x1_d16", "small_2x512x4_d64"):
        c = gi.WORKLOADS[name]
        inp = gi.make_chunk_inputs(c["B"], c["T"], c["H"], c["dk"], c["dv"], c["dtype"],
                                   c["seed"], s0=c["s0"])
        args = [inp[x].double().numpy() for x in ("q", "k", "v", "alpha", "b", "w")]
        S0 = inp["S0"].double().numpy()
        o, Sf = oracle.fwd(*args, S0=S0)
        o2, Sf2 = reference_np.fwd(*args, S0=S0)
        assert rel(o, o2) < 1e-12 and rel(Sf, Sf2) < 1e-12


def test_kda_reduction_on_small_workload():
    """The small workload with b = w = beta (scalar per batch, token, head): the GDN-2
    oracle equals textbook KDA on every head."""
    c = gi.WORKLOADS["small_2x512x4_d64"]
    inp = gi.make_chunk_inputs(c["B"], 128, c["H"], c["dk"], c["dv"], "f32", c["seed"],
                               s0="normal", scalar_beta=True)
    A = {x: inp[x].double().numpy() for x in ("q", "k", "v", "alpha", "b", "w")}
    S0 = inp["S0"].double().numpy()
    o, Sf = oracle.fwd(*(A[x] for x in ("q", "k", "v", "alpha", "b", "w")), S0=S0)
    for n in range(c["B"]):
        for h in range(c["H"]):
            oref, Sref = pins.kda_textbook(A["q"][n, :, h], A["k"][n, :, h], A["v"][n, :, h],
                                           A["alpha"][n, :, h], A["b"][n, :, h, 0], S0[n, h])
            assert rel(o[n, :, h], oref) < 1e-12 and rel(Sf[n, h], Sref) < 1e-12


def test_nan_propagates():
    rng = np.random.default_rng(5)
    q, k, v, alpha, b, w, S0 = rand_head(rng, 10, 8, 8)
    v[4, 3] = np.nan
    o, Sf = run_head(q, k, v, alpha, b, w, S0)
    assert np.all(np.isfinite(o[:4])) and np.isnan(o[4:]).any() and np.isnan(Sf).any()


# ---------------------------------------------- the pins catch mistakes --
def _pin_suite_passes(mutation):
    """Run the pins above on the NumPy transcription with one planted
    mistake; return False as soon as one of them fails."""
    rng = np.random.default_rng(99)
    T, d = 24, 8
    q, k, v, alpha, b, w, S0 = rand_head(rng, T, d, d)
    f = lambda *a, **kw: reference_np.fwd_head(*a, mutation=mutation, **kw)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    B1 = np.repeat(beta[:, None], d, 1)
    checks = []
    o, S = f(q, k, v, alpha, B1, B1, S0)
    oref, Sref = pins.kda_textbook(q, k, v, alpha, beta, S0)
    checks.append(rel(o, oref) < 1e-10 and rel(S, Sref) < 1e-10)
    o, _ = f(q, k, v, np.ones((T, d)), np.zeros((T, d)), np.ones((T, d)), S0)
    checks.append(rel(o, pins.linear_attention_closed(q, k, v, S0)) < 1e-10)
    o, _ = f(q, k, v, alpha, np.zeros((T, d)), np.ones((T, d)), S0)
    checks.append(rel(o, pins.decayed_linear_closed(q, k, v, alpha, S0)) < 1e-10)
    o, _ = f(k, k, v, alpha, np.ones((T, d)), w, S0)
    checks.append(np.allclose(o, w * v, atol=1e-10))
    g = _parse_golden()
    o, S = f(g["q"], g["k"], g["v"], g["alpha"], g["b"], g["w"], g["S0"].reshape(2, 2))
    checks.append(np.array_equal(o, g["R5.o"]) and np.array_equal(S.ravel(), g["R5.S_final"].ravel()))
    return all(checks)


@pytest.mark.parametrize("mutation", ["no_b_in_read", "gated_write_key", "decay_after",
                                      "read_before", "decay_value_axis", "transpose_read",
                                      "swap_gates", "w_on_delta", "sign_write"])
def test_pins_catch_planted_mistakes(mutation):
    assert _pin_suite_passes(None)
    assert not _pin_suite_passes(mutation)


# ------------------------------------------------------------ layer prep
# Pins of the float64 layer prep (oracle/layer_prep.py) by properties its
# definitions fix, not by re-evaluating them.
def test_layer_prep_l2_normalise_properties():
    from oracle import layer_prep as lp
    rng = np.random.default_rng(11)
    x = rng.normal(size=(3, 5, 7, 32)) * rng.uniform(0.1, 10.0, size=(3, 5, 7, 1))
    y = lp.l2_normalise(x)
    assert np.allclose(np.sum(y * y, axis=-1), 1.0, atol=1e-13)          # unit length
    assert np.allclose(lp.l2_normalise(4.5 * x), y, atol=1e-15)          # scale invariant
    assert np.all(np.sum(y * x, axis=-1) > 0)                            # same direction
    e = np.zeros(8); e[3] = -2.0
    assert np.array_equal(lp.l2_normalise(e), -np.eye(8)[3])            # a basis vector
    assert np.array_equal(lp.l2_normalise(np.zeros(8)), np.zeros(8))    # zero stays zero


def test_layer_prep_sigmoid_properties():
    from oracle import layer_prep as lp
    x = np.linspace(-30, 30, 601)
    s = lp.sigmoid(x)
    assert lp.sigmoid(0.0) == 0.5
    assert np.allclose(s + lp.sigmoid(-x), 1.0, atol=1e-15)              # symmetry
    assert np.all(np.diff(s) > 0) and s.min() > 0 and s.max() < 1       # monotone into (0, 1)
    p = np.array([0.1, 0.25, 0.9])
    assert np.allclose(lp.sigmoid(np.log(p / (1 - p))), p, atol=1e-15)  # inverse of the logit
    # derivative s(1 - s) against a central difference
    h = 1e-6
    d = (lp.sigmoid(x + h) - lp.sigmoid(x - h)) / (2 * h)
    assert np.allclose(d, s * (1 - s), atol=1e-9)


def test_layer_prep_decay_properties():
    from oracle import layer_prep as lp
    g = -np.array([0.0, 0.01, 0.5, 3.0])
    a = lp.decay_from_log(g)
    assert a[0] == 1.0
    assert np.allclose(np.log(a), g, atol=1e-15)
    # products of decays are sums of their logs
    assert np.isclose(lp.decay_from_log(g[1] + g[2]), a[1] * a[2], rtol=1e-15)


def test_layer_prep_feeds_the_recurrence():
    """Raw inputs that are already normalised (to float32 rounding), with
    gate logits and log decay of known values, reproduce the recurrence on
    the plain inputs (to that rounding)."""
    from oracle import layer_prep as lp
    inp = gi.make_chunk_inputs(1, 40, 2, 16, 16, "f32", seed=12, s0="normal")
    b = inp["b"].double().numpy(); w = inp["w"].double().numpy(); al = inp["alpha"].double().numpy()
    raw = lp.layer_prep(inp["q"], inp["k"], np.log(al), np.log(b / (1 - b)), np.log(w / (1 - w)))
    o1, S1 = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["b"], inp["w"], S0=inp["S0"])
    o2, S2 = oracle.fwd(raw["q"], raw["k"], inp["v"], raw["alpha"], raw["b"], raw["w"], S0=inp["S0"])
    assert np.abs(o1 - o2).max() <= 1e-6 * np.abs(o1).max()
    assert np.abs(S1 - S2).max() <= 1e-6 * np.abs(S1).max()


@pytest.mark.parametrize("dk,dv", [(3, 5), (6, 2)])
@pytest.mark.parametrize("rule", ["R5", "R1"])
def test_P9_rectangular_head_equals_widened_square(dk, dv, rule):
    """A head with dk != dv gives what the square head of width
    d = max(dk, dv) gives on widened inputs (extra key channels: q = k = b = 0,
    alpha = 1; extra value channels: v = w = 0), on its dk x dv corner; the
    widened rows and columns of the square state and the widened outputs stay
    exactly zero.  A dk/dv index swapped anywhere in the oracle breaks it."""
    inp = gi.make_chunk_inputs(2, 9, 2, dk, dv, "f32", seed=61 + dk, s0="normal")
    d = max(dk, dv)

    def widen(x, width, fill):
        out = torch.full(x.shape[:-1] + (d,), fill, dtype=torch.float64)
        out[..., :width] = x.double()
        return out

    wide = {"q": widen(inp["q"], dk, 0.0), "k": widen(inp["k"], dk, 0.0), "alpha": widen(inp["alpha"], dk, 1.0),
            "b": widen(inp["b"], dk, 0.0), "v": widen(inp["v"], dv, 0.0), "w": widen(inp["w"], dv, 0.0)}
    S0 = torch.zeros(inp["S0"].shape[:2] + (d, d), dtype=torch.float64)
    S0[:, :, :dk, :dv] = inp["S0"].double()
    names = ("q", "k", "v", "alpha", "b", "w")
    o_r, S_r = oracle.fwd(*(inp[n] for n in names), S0=inp["S0"], rule=rule)
    o_s, S_s = oracle.fwd(*(wide[n] for n in names), S0=S0, rule=rule)
    assert o_r.shape[-1] == dv and S_r.shape[-2:] == (dk, dv)
    np.testing.assert_allclose(o_r, o_s[..., :dv], rtol=0, atol=1e-12)
    np.testing.assert_allclose(S_r, S_s[:, :, :dk, :dv], rtol=0, atol=1e-12)
    assert np.all(o_s[..., dv:] == 0) and np.all(S_s[:, :, dk:, :] == 0) and np.all(S_s[:, :, :, dv:] == 0)
