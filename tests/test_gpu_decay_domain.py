"""GPU parity at the edge of the decay's range (MI355X only): strong
per-channel decay, decays of 1e-4 and below, and alpha = 0 exactly, on the
chunked forward (every path), the segment maps, layer prep (log-decay down
to -20 and -inf) and the backward.  The pages keep the log-decay in float32
because the in-chunk cumulative sum is precision-sensitive (aixai.ru blog,
section on how the method is implemented in practice); the kernels form
every decay factor as a sum of log decays (never a difference of two) and
take the diagonal 16-token blocks pair by pair when a sub-block decays by
more than 2^-64, so any decay, zero included, is exact to rounding.
Tolerances as everywhere: max |x - ref| / max |ref| <= 1e-4 (float32
inputs), 2e-2 (bfloat16)."""
import numpy as np
import pytest
import torch

import gdn2_inputs as gi
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("q", "k", "v", "alpha", "b", "w")
GRADS = ("dq", "dk", "dv", "dalpha", "db", "dw")

# strong: decay logits ~ N(-2, 2^2), 1% of the decays 1e-4 and 1% zero;
# spiky: the default decay (logits ~ N(3, 1)) with 0.5% of the decays 1e-6
# and 0.5% zero, so that most 16-token sub-blocks keep the matrix-core
# diagonal and a few take the pairwise one
KINDS = {"strong": dict(logit_mean=-2.0, logit_std=2.0, tiny_frac=0.01, tiny=1e-4, zero_frac=0.01),
         "spiky": dict(logit_mean=3.0, logit_std=1.0, tiny_frac=0.005, tiny=1e-6, zero_frac=0.005)}


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_07_amd as mod
    mod.lib()
    return mod


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def check(pairs, tol, label):
    for name, x, ref in pairs:
        assert np.isfinite(x).all(), f"{label}: {name} has non-finite values"
        e = rel_err(x, ref)
        print(f"{label} {name} err={e:.3e}", flush=True)
        assert e <= tol, f"{label}: {name} error {e:.3e} > {tol}"


def gpu_fwd(g, inp, chunk, cu=None, path="auto", layer_prep=False):
    d = {n: inp[n].cuda() for n in NAMES}
    S0 = inp.get("S0")
    o, Sf = g.chunk_fwd(*(d[n] for n in NAMES), S0=None if S0 is None else S0.cuda(),
                        cu_seqlens=None if cu is None else cu.cuda(), chunk=chunk, path=path,
                        layer_prep=layer_prep)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), Sf.cpu().numpy()


FWD_CASES = [  # dtype, d, chunk, T, path
    ("f32", 64, 64, 200, "two_pass"),
    ("f32", 64, 16, 77, "two_pass"),
    ("f32", 32, 16, 130, "fused"),
    ("bf16", 128, 64, 200, "two_pass"),
    ("bf16", 128, 64, 200, "fused"),
    ("bf16", 64, 16, 150, "two_pass"),
    ("bf16", 16, 64, 90, "two_pass"),
]


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("dtype,d,chunk,T,path", FWD_CASES)
def test_forward_strong_decay(g, kind, dtype, d, chunk, T, path):
    inp = gi.make_strong_decay_inputs(2, T, 3, d, d, dtype, seed=700 + d + T, s0="normal", **KINDS[kind])
    a = inp["alpha"].float().numpy()
    print(f"case fwd {kind} {dtype} d={d} C={chunk} T={T} {path}: alpha min {a.min():.1e}, "
          f"zeros {int((a == 0).sum())}", flush=True)
    o, Sf = gpu_fwd(g, inp, chunk, path=path)
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    check((("o", o, o_ref), ("S_final", Sf, S_ref)), TOL[dtype], f"fwd {kind} {dtype} d={d} C={chunk} {path}")


def test_forward_strong_decay_packed_and_segments(g):
    """Packed input with an empty sequence, and one long sequence on the
    default path (the segment schedule: maps, their scan, re-runs)."""
    lens = [70, 0, 1, 130, 45]
    cu = gi.cu_seqlens_from(lens)
    inp = gi.make_strong_decay_inputs(1, sum(lens), 2, 64, 64, "f32", seed=731, s0="normal",
                                      num_seqs=len(lens), **KINDS["strong"])
    print("case fwd strong packed", flush=True)
    o, Sf = gpu_fwd(g, inp, 16, cu=cu)
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"], cu_seqlens=cu)
    check((("o", o, o_ref), ("S_final", Sf, S_ref)), TOL["f32"], "fwd strong packed")
    inp = gi.make_strong_decay_inputs(1, 130 * 64 + 5, 2, 32, 32, "f32", seed=732, s0="normal", **KINDS["spiky"])
    print("case fwd spiky segment schedule", flush=True)
    o, Sf = gpu_fwd(g, inp, 64)
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    check((("o", o, o_ref), ("S_final", Sf, S_ref)), TOL["f32"], "fwd spiky segment schedule")


def test_forward_all_zero_decay(g):
    """alpha = 0 everywhere: every token starts from an erased state, so
    o_t = (w_t (.) v_t) (k_t . q_t) and S_final = k_T (w_T (.) v_T)^T."""
    inp = gi.make_chunk_inputs(1, 100, 2, 32, 32, "f32", seed=733, s0="normal")
    inp["alpha"] = torch.zeros_like(inp["alpha"])
    print("case fwd alpha = 0", flush=True)
    o, Sf = gpu_fwd(g, inp, 64, path="two_pass")
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    check((("o", o, o_ref), ("S_final", Sf, S_ref)), TOL["f32"], "fwd alpha = 0")


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("dtype,d,chunk,T", [("f32", 32, 64, 190), ("f32", 64, 16, 77), ("bf16", 128, 64, 300)])
def test_segment_map_strong_decay(g, kind, dtype, d, chunk, T):
    inp = gi.make_strong_decay_inputs(2, T, 2, d, d, dtype, seed=740 + d, **KINDS[kind])
    print(f"case map {kind} {dtype} d={d} C={chunk} T={T}", flush=True)
    dd = {n: inp[n].cuda() for n in NAMES}
    Phi, Psi = g.segment_map(*(dd[n] for n in NAMES), chunk=chunk)
    torch.cuda.synchronize()
    rPhi, rPsi = oracle.segment_map(*(inp[n] for n in NAMES))
    check((("Phi", Phi.cpu().numpy(), rPhi), ("Psi", Psi.cpu().numpy(), rPsi)), TOL[dtype],
          f"map {kind} {dtype} d={d} C={chunk}")


@pytest.mark.parametrize("path", ["two_pass", "fused"])
@pytest.mark.parametrize("dtype,d,chunk,T", [("f32", 64, 64, 190), ("bf16", 128, 64, 200), ("bf16", 64, 16, 77)])
def test_layer_prep_log_decay_to_minus_20(g, dtype, d, chunk, T, path):
    """Layer prep with the float32 log-decay down to -20 and 0.5% of it at
    -inf (alpha = 0)."""
    from oracle import layer_prep as lp
    raw = gi.make_layer_inputs(2, T, 3, d, d, dtype, seed=750 + T, s0="normal", strong_decay=True,
                               neg_inf_frac=0.005)
    print(f"case layer prep strong {dtype} d={d} C={chunk} {path}", flush=True)
    prep = lp.layer_prep(raw["q"], raw["k"], raw["alpha"], raw["b"], raw["w"])
    o_ref, S_ref = oracle.fwd(prep["q"], prep["k"], raw["v"], prep["alpha"], prep["b"], prep["w"], S0=raw["S0"])
    o, Sf = gpu_fwd(g, raw, chunk, path=path, layer_prep=True)
    check((("o", o, o_ref), ("S_final", Sf, S_ref)), TOL[dtype], f"layer prep strong {dtype} d={d} {path}")


# ------------------------------------------------------------- backward
def gpu_bwd(g, inp, grads, chunk, layer_prep=False):
    d = {n: inp[n].cuda() for n in NAMES}
    S0 = inp.get("S0")
    out = g.chunk_bwd(*(d[n] for n in NAMES), grads["dout"].cuda(), S0=None if S0 is None else S0.cuda(),
                      dS_final=grads["dS_final"].cuda(), chunk=chunk, layer_prep=layer_prep)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() for k, v in out.items() if v is not None}


@pytest.mark.parametrize("dtype,d,chunk,T", [("f32", 64, 64, 190), ("f32", 32, 16, 77), ("bf16", 128, 64, 200),
                                             ("bf16", 64, 16, 150)])
def test_backward_strong_decay_log_input(g, dtype, d, chunk, T):
    """Backward with the float32 log-decay input (layer prep) down to -20
    and 0.5% at -inf: every gradient, dL/d(ln alpha) included, and dS0."""
    from oracle import layer_prep as lp
    raw = gi.make_layer_inputs(2, T, 3, d, d, dtype, seed=760 + T, s0="normal", strong_decay=True,
                               neg_inf_frac=0.005)
    grads = gi.make_bwd_grads(2, T, 3, d, d, dtype, seed=760 + T)
    print(f"case bwd layer prep strong {dtype} d={d} C={chunk}", flush=True)
    got = gpu_bwd(g, raw, grads, chunk, layer_prep=True)
    prep = lp.layer_prep(raw["q"], raw["k"], raw["alpha"], raw["b"], raw["w"])
    gp = oracle.bwd(prep["q"], prep["k"], raw["v"], prep["alpha"], prep["b"], prep["w"], grads["dout"],
                    S0=raw["S0"], dS_final=grads["dS_final"])
    ref = lp.layer_prep_bwd(raw["q"], raw["k"], raw["alpha"], raw["b"], raw["w"], gp)
    ref["dS0"] = gp["dS0"]
    check([(n, got[n], ref[n]) for n in GRADS + ("dS0",)], TOL[dtype], f"bwd layer prep strong {dtype} d={d}")


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("dtype,d,chunk,T", [("f32", 64, 64, 190), ("bf16", 128, 64, 200), ("bf16", 32, 16, 77)])
def test_backward_strong_decay(g, kind, dtype, d, chunk, T):
    """Backward with alpha itself as input, decays down to 1e-6 and zero:
    dq, dk, dv, db, dw and dS0 everywhere.  dL/dalpha is formed as
    dL/d(ln alpha) / alpha, whose absolute error grows as 1 / alpha, so it is
    compared where alpha >= 0.05 (as alpha * dL/dalpha = dL/d(ln alpha)
    everywhere it is finite); alpha = 0 has no log and gives no finite
    dL/dalpha on this input form (the log-decay input above covers it)."""
    inp = gi.make_strong_decay_inputs(2, T, 3, d, d, dtype, seed=770 + d + T, s0="normal", **KINDS[kind])
    grads = gi.make_bwd_grads(2, T, 3, d, d, dtype, seed=770 + d + T)
    print(f"case bwd {kind} {dtype} d={d} C={chunk}", flush=True)
    got = gpu_bwd(g, inp, grads, chunk)
    ref = oracle.bwd(*(inp[n] for n in NAMES), grads["dout"], S0=inp["S0"], dS_final=grads["dS_final"])
    check([(n, got[n], ref[n]) for n in ("dq", "dk", "dv", "db", "dw", "dS0")], TOL[dtype],
          f"bwd {kind} {dtype} d={d}")
    a = inp["alpha"].float().numpy()
    big = a >= 0.05
    e = rel_err(got["dalpha"][big], ref["dalpha"][big])
    print(f"bwd {kind} {dtype} d={d} dalpha (alpha >= 0.05) err={e:.3e}", flush=True)
    assert e <= TOL[dtype]
    pos = a > 0
    e = rel_err(got["dalpha"][pos] * a[pos], ref["dalpha"][pos] * a[pos])
    print(f"bwd {kind} {dtype} d={d} alpha dalpha (alpha > 0) err={e:.3e}", flush=True)
    assert e <= TOL[dtype]
