"""GPU parity of libgdn2 against the float64 CPU oracle (MI355X only).

Every case runs the HIP kernels through the C ABI (via the thin Python
binding) on seeded synthetic inputs and compares element by element with the
oracle on the same stored inputs.  Tolerances (max |x - ref| / max |ref| per
tensor): 1e-4 for float32 inputs, 2e-2 for bfloat16 inputs, for o and
S_final separately.
"""
import numpy as np
import pytest
import torch

import gdn2_inputs as gi
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("q", "k", "v", "alpha", "b", "w")


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


def to_dev(inp):
    return {kk: (vv.cuda() if isinstance(vv, torch.Tensor) else vv) for kk, vv in inp.items()}


def gpu_fwd(g, inp, chunk, cu=None, recurrent=False, S0=None, path="auto", layer_prep=False):
    d = to_dev(inp)
    o, Sf = g.chunk_fwd(*(d[n] for n in NAMES), S0=(S0.cuda() if S0 is not None else d.get("S0")),
                        cu_seqlens=None if cu is None else cu.cuda(), chunk=chunk, recurrent=recurrent,
                        path=path, layer_prep=layer_prep)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), Sf.cpu().numpy()


def check(o, Sf, o_ref, S_ref, tol, label=""):
    eo, es = rel_err(o, o_ref), rel_err(Sf, S_ref)
    print(f"{label} err_o={eo:.3e} err_S={es:.3e}", flush=True)
    assert eo <= tol, f"{label}: o error {eo:.3e} > {tol}"
    assert es <= tol, f"{label}: S_final error {es:.3e} > {tol}"


def make(name, **over):
    c = dict(gi.WORKLOADS[name])
    c.update(over)
    return c, gi.make_chunk_inputs(c["B"], c["T"], c["H"], c["dk"], c["dv"], c["dtype"], c["seed"],
                                   s0=c["s0"])


# ---------------------------------------------------------- small workloads
@pytest.mark.parametrize("recurrent", [False, True])
def test_tiny_1x64x1(g, recurrent):
    c, inp = make("tiny_1x64x1_d16")
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    for s0 in (inp["S0"], None):  # explicit zeros and NULL
        inp2 = dict(inp, S0=s0)
        o, Sf = gpu_fwd(g, inp2, c["chunk"], recurrent=recurrent)
        check(o, Sf, o_ref, S_ref, TOL["f32"], f"tiny rec={recurrent} s0={'zeros' if s0 is not None else 'NULL'}")


@pytest.mark.parametrize("path", ["auto", "recurrent", "two_pass", "fused"])
def test_small_2x512x4(g, path):
    c, inp = make("small_2x512x4_d64")
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    o, Sf = gpu_fwd(g, inp, c["chunk"], path=path)
    check(o, Sf, o_ref, S_ref, TOL["f32"], f"small {path}")


def test_small_collapsed_gates(g):
    """b = w = beta (KDA case): the GPU matches the oracle, which is pinned to
    textbook KDA on the CPU."""
    c = gi.WORKLOADS["small_2x512x4_d64"]
    inp = gi.make_chunk_inputs(c["B"], c["T"], c["H"], c["dk"], c["dv"], "f32", c["seed"],
                               s0="normal", scalar_beta=True)
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    o, Sf = gpu_fwd(g, inp, 64)
    check(o, Sf, o_ref, S_ref, TOL["f32"], "small collapsed gates")


RAGGED = [("bf16", 128, 64, 200), ("bf16", 64, 16, 77), ("f32", 128, 64, 130), ("f32", 32, 64, 64),
          ("bf16", 16, 16, 33), ("f32", 64, 16, 1), ("bf16", 128, 16, 45), ("f32", 64, 64, 190),
          ("f32", 128, 16, 40)]


@pytest.mark.parametrize("path", ["two_pass", "fused"])
@pytest.mark.parametrize("dtype,d,chunk,T", RAGGED)
def test_ragged_shapes(g, dtype, d, chunk, T, path):
    fused_ok = (chunk == 16 or d in (64, 128)) and not (dtype == "f32" and d == 128 and chunk == 64)
    if path == "fused" and not fused_ok:
        with pytest.raises(g.Gdn2Error):
            gpu_fwd(g, gi.make_chunk_inputs(1, 16, 1, d, d, dtype, seed=1), chunk, path=path)
        return
    inp = gi.make_chunk_inputs(2, T, 3, d, d, dtype, seed=100 + T, s0="normal")
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    o, Sf = gpu_fwd(g, inp, chunk, path=path)
    check(o, Sf, o_ref, S_ref, TOL[dtype], f"ragged {path} {dtype} d={d} C={chunk} T={T}")


# The state scan splits the dv columns of a head over 1, 2 or 4 tiles per
# workgroup depending on how many (sequence, head) units there are: these
# batch sizes land in each of the three splits (d = 128: <= 32 / <= 64 / more
# units; d = 64: <= 64 / <= 128 / more).
SPLITS = [("bf16", 128, 2), ("bf16", 128, 3), ("bf16", 128, 5), ("f32", 64, 4), ("f32", 64, 6),
          ("f32", 64, 9)]


@pytest.mark.parametrize("dtype,d,B", SPLITS)
def test_scan_column_splits(g, dtype, d, B):
    inp = gi.make_chunk_inputs(B, 150, 16, d, d, dtype, seed=300 + B, s0="normal")
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    o, Sf = gpu_fwd(g, inp, 64, path="two_pass")
    check(o, Sf, o_ref, S_ref, TOL[dtype], f"split {dtype} d={d} units={16 * B}")


# Gates given per (token, head) ([B, T, H]) instead of per channel: the GPU
# reads the compact tensors, the oracle gets the same values repeated over the
# channels.  kda: b = w = beta; gdn: plus a per-(token, head) alpha; b_only /
# w_only: the single-gate ablations.
GATE_CASES = {"kda": ("b", "w"), "gdn": ("b", "w", "alpha"), "b_only": ("b",), "w_only": ("w",)}


@pytest.mark.parametrize("path", ["two_pass", "fused"])
@pytest.mark.parametrize("dtype,d,T", [("f32", 64, 190), ("bf16", 128, 200)])
@pytest.mark.parametrize("case", list(GATE_CASES))
def test_per_token_gates(g, case, dtype, d, T, path):
    inp = gi.make_chunk_inputs(2, T, 3, d, d, dtype, seed=400 + T, s0="normal",
                               scalar_beta=(case in ("kda", "gdn")))
    full, compact = dict(inp), dict(inp)
    for x in GATE_CASES[case]:
        s = inp[x][..., 0].contiguous()           # one value per (batch, token, head)
        compact[x] = s
        full[x] = s[..., None].expand_as(inp[x]).contiguous()
    o_ref, S_ref = oracle.fwd(*(full[n] for n in NAMES), S0=inp["S0"])
    o, Sf = gpu_fwd(g, compact, 64, path=path)
    check(o, Sf, o_ref, S_ref, TOL[dtype], f"gates {case} {path} {dtype} d={d}")


@pytest.mark.parametrize("case", list(GATE_CASES))
def test_per_token_gates_segment_schedule(g, case):
    """Per-(token, head) gates on the default path of two sequences of 130
    chunks and 3 heads, which takes the segment schedule (the gate layouts
    reach the maps and the re-runs)."""
    B, T, H, d = 2, 130 * 64 + 9, 3, 32
    inp = gi.make_chunk_inputs(B, T, H, d, d, "f32", seed=71, s0="normal", alpha_mean=8.0,
                               scalar_beta=(case in ("kda", "gdn")))
    full, compact = dict(inp), dict(inp)
    for x in GATE_CASES[case]:
        s = inp[x][..., 0].contiguous()
        compact[x] = s
        full[x] = s[..., None].expand_as(inp[x]).contiguous()
    print(f"case gates {case} segment schedule T={T}", flush=True)
    o_ref, S_ref = oracle.fwd(*(full[n] for n in NAMES), S0=inp["S0"])
    o, Sf = gpu_fwd(g, compact, 64)
    check(o, Sf, o_ref, S_ref, TOL["f32"], f"gates {case} segment schedule")


def test_per_token_gates_rejected_on_recurrent_path(g):
    inp = gi.make_chunk_inputs(1, 32, 1, 16, 16, "f32", seed=5)
    inp["b"] = inp["b"][..., 0].contiguous()
    with pytest.raises(g.Gdn2Error):
        gpu_fwd(g, inp, 16, recurrent=True)


# Layer prep: raw q, k (not normalised), gate logits and the float32
# natural-log decay go in; the oracle applies the float64 layer prep
# (oracle/layer_prep.py) to the same stored values and runs the recurrence.
@pytest.mark.parametrize("path", ["two_pass", "fused"])
@pytest.mark.parametrize("dtype,d,chunk,T", [("f32", 64, 64, 190), ("bf16", 128, 64, 200), ("bf16", 64, 16, 77)])
@pytest.mark.parametrize("scalar", [False, True])
def test_layer_prep(g, dtype, d, chunk, T, path, scalar):
    from oracle import layer_prep as lp
    raw = gi.make_layer_inputs(2, T, 3, d, d, dtype, seed=500 + T, s0="normal", scalar_beta=scalar)
    prep = lp.layer_prep(raw["q"], raw["k"], raw["alpha"], raw["b"], raw["w"])
    full = {x: (prep[x][..., None] * np.ones(d) if prep[x].ndim == 3 else prep[x])
            for x in ("q", "k", "alpha", "b", "w")}
    o_ref, S_ref = oracle.fwd(full["q"], full["k"], raw["v"], full["alpha"], full["b"], full["w"], S0=raw["S0"])
    o, Sf = gpu_fwd(g, raw, chunk, path=path, layer_prep=True)
    check(o, Sf, o_ref, S_ref, TOL[dtype], f"layer prep {path} {dtype} d={d} C={chunk} scalar={scalar}")


def test_layer_prep_rejected_on_recurrent_path(g):
    raw = gi.make_layer_inputs(1, 32, 1, 16, 16, "f32", seed=6)
    with pytest.raises(g.Gdn2Error):
        gpu_fwd(g, raw, 16, recurrent=True, layer_prep=True)


def test_chunk_size_invariance(g):
    inp = gi.make_chunk_inputs(1, 256, 2, 64, 64, "f32", seed=7, s0="normal")
    o16, S16 = gpu_fwd(g, inp, 16)
    o64, S64 = gpu_fwd(g, inp, 64)
    orec, Srec = gpu_fwd(g, inp, 64, recurrent=True)
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    for o, S, lab in ((o16, S16, "C16"), (o64, S64, "C64"), (orec, Srec, "rec")):
        check(o, S, o_ref, S_ref, TOL["f32"], lab)


def test_erase_gate_up_to_two(g):
    """b in [0, 2] (the extended erase range): nothing is clamped."""
    inp = gi.make_chunk_inputs(1, 128, 2, 64, 64, "f32", seed=8, s0="normal")
    inp["b"] = (inp["b"] * 2.0).contiguous()
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    o, Sf = gpu_fwd(g, inp, 64)
    check(o, Sf, o_ref, S_ref, TOL["f32"], "b*2")


# ----------------------------------------------------------- packed input
def test_packed_small_with_empty_sequences(g):
    lens = [70, 0, 1, 64, 130, 0, 15]
    cu = gi.cu_seqlens_from(lens)
    T = int(cu[-1])
    inp = gi.make_chunk_inputs(1, T, 2, 64, 64, "f32", seed=9, s0="normal", num_seqs=len(lens))
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"], cu_seqlens=cu)
    for chunk in (16, 64):
        for path in ("two_pass", "fused"):
            o, Sf = gpu_fwd(g, inp, chunk, cu=cu, path=path)
            check(o, Sf, o_ref, S_ref, TOL["f32"], f"packed C={chunk} {path}")
    o, Sf = gpu_fwd(g, inp, 64, cu=cu, recurrent=True)
    check(o, Sf, o_ref, S_ref, TOL["f32"], "packed rec")


def test_packed_32768_all_sequences(g):
    """32768 packed tokens (10 sequences of lengths uniform in [256, 8192]),
    H=16, d=128, bf16, in the benchmark's launch configuration: every output
    element and every sequence's final state against the oracle."""
    lens = gi.packed_lengths(3)
    cu = gi.cu_seqlens_from(lens)
    c = gi.WORKLOADS["packed_32768x16_d128"]
    inp = gi.make_chunk_inputs(1, c["T"], c["H"], c["dk"], c["dv"], "bf16", c["seed"], s0=None,
                               num_seqs=len(lens))
    print(f"case packed 32768 lens={lens}", flush=True)
    o, Sf = gpu_fwd(g, inp, 64, cu=cu)
    o_ref, S_ref = oracle.fwd(*(inp[x] for x in NAMES), cu_seqlens=cu)
    check(o, Sf, o_ref, S_ref, TOL["bf16"], "packed 32768, all sequences")
    for n in range(len(lens)):  # and per sequence, against its own scale
        a, bnd = int(cu[n]), int(cu[n + 1])
        check(o[:, a:bnd], Sf[n:n + 1], o_ref[:, a:bnd], S_ref[n:n + 1], TOL["bf16"], f"packed seq{n} len={bnd - a}")


def test_varlen_equals_separate_runs(g):
    lens = [100, 37, 64]
    cu = gi.cu_seqlens_from(lens)
    inp = gi.make_chunk_inputs(1, int(cu[-1]), 2, 128, 128, "bf16", seed=10, s0="normal",
                               num_seqs=3)
    o, Sf = gpu_fwd(g, inp, 64, cu=cu)
    for n in range(3):
        a, bnd = int(cu[n]), int(cu[n + 1])
        sub = {x: inp[x][:, a:bnd].contiguous() for x in NAMES}
        sub["S0"] = inp["S0"][n:n + 1].contiguous()
        o1, S1 = gpu_fwd(g, sub, 64)
        np.testing.assert_array_equal(o[:, a:bnd], o1)
        np.testing.assert_array_equal(Sf[n:n + 1], S1)


@pytest.mark.parametrize("path", ["two_pass", "fused", "recurrent"])
def test_chunk_aligned_slices_chain_exactly(g, path):
    """Cutting every sequence at chunk boundaries and running the pieces in
    order, each from the state the previous piece left, reproduces the
    whole-sequence outputs and final state bit for bit: the kernels carry
    the state from chunk to chunk in float32, as S0 is read and S_final
    written.  The last piece ends in a ragged chunk."""
    B, T, H, d, C = 2, 450, 3, 128, 64
    inp = gi.make_chunk_inputs(B, T, H, d, d, "bf16", seed=23, s0="normal")
    print(f"case path={path} B={B} T={T} H={H} d={d}", flush=True)
    o, Sf = gpu_fwd(g, inp, C, path=path)
    S = inp["S0"]
    cuts = [0, 128, 192, T]
    for a, bnd in zip(cuts[:-1], cuts[1:]):
        sub = {x: inp[x][:, a:bnd].contiguous() for x in NAMES}
        o1, S1 = gpu_fwd(g, sub, C, S0=S, path=path)
        np.testing.assert_array_equal(o[:, a:bnd], o1)
        S = torch.from_numpy(S1)
    np.testing.assert_array_equal(Sf, S.numpy())


# -------------------------------------------------------- headline config
@pytest.fixture(scope="module")
def layer_case():
    """The layer workload (B=8, T=4096, H=16, d=128, bf16) and the oracle's
    output for all of it (128 (batch, head) units, float64)."""
    c, inp = make("layer_8x4096x16_d128")
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES))
    return inp, o_ref, S_ref


@pytest.mark.parametrize("path", ["auto", "two_pass"])
def test_layer_8x4096x16_all_units(g, layer_case, path):
    """The layer workload at full size in the launch configuration the
    benchmark times ("auto") and on the forced two-pass kernels: every
    element of o and S_final against the oracle, over the whole tensor and
    per (batch, head) unit against that unit's own scale."""
    inp, o_ref, S_ref = layer_case
    print(f"case layer 8x4096x16 path={path}", flush=True)
    o, Sf = gpu_fwd(g, inp, 64, path=path)
    check(o, Sf, o_ref, S_ref, TOL["bf16"], f"layer {path}")
    worst_o = max(rel_err(o[bb, :, hh], o_ref[bb, :, hh]) for bb in range(8) for hh in range(16))
    worst_S = max(rel_err(Sf[bb, hh], S_ref[bb, hh]) for bb in range(8) for hh in range(16))
    print(f"layer {path}: worst unit err_o={worst_o:.3e} err_S={worst_S:.3e}", flush=True)
    assert worst_o <= TOL["bf16"] and worst_S <= TOL["bf16"]


@pytest.mark.parametrize("T", [2048, 4096, 8192, 16384, 32768])
def test_sweep_all_units(g, T):
    """T sweep at B*T = 32768 (B = 32768 / T sequences of 16 heads, d=128,
    bf16) on the default path, as the benchmark runs it (the 32768 point
    takes the segment schedule): every element against the oracle."""
    B = 32768 // T
    inp = gi.make_chunk_inputs(B, T, 16, 128, 128, "bf16", seed=30 + B, s0=None)
    print(f"case sweep T={T} B={B}", flush=True)
    o, Sf = gpu_fwd(g, inp, 64)
    o_ref, S_ref = oracle.fwd(*(inp[x] for x in NAMES))
    check(o, Sf, o_ref, S_ref, TOL["bf16"], f"sweep T={T}")


@pytest.mark.parametrize("dtype,d,B,H,T", [("f32", 64, 1, 2, 512 * 64 + 100), ("bf16", 128, 1, 4, 512 * 64 + 37),
                                           ("bf16", 64, 1, 16, 130 * 64 + 5), ("bf16", 64, 2, 4, 130 * 64 + 5),
                                           ("f32", 32, 4, 2, 160 * 64 - 3), ("bf16", 64, 2, 16, 130 * 64 + 5),
                                           ("f32", 32, 1, 32, 128 * 64 + 9)])
def test_long_sequence_segment_schedule(g, dtype, d, B, H, T):
    """Sequences of 128 chunks or more with at most 32 (sequence, head)
    units on the default path: the library cuts every sequence into 4, 8 or
    16 segments (maps of all but the last, the scan of each sequence's maps,
    every segment's scan from its entering state, S_final from the last).
    Checked against the oracle with initial states, ragged last segments,
    and S_final written over S0."""
    inp = gi.make_chunk_inputs(B, T, H, d, d, dtype, seed=41 + d + B, s0="normal", alpha_mean=8.0)
    print(f"case segment schedule {dtype} d={d} B={B} H={H} T={T}", flush=True)
    dd = to_dev(inp)
    S = dd["S0"].clone()
    o, _ = g.chunk_fwd(*(dd[n] for n in NAMES), S0=S, S_final=S, chunk=64)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    check(o.float().cpu().numpy(), S.cpu().numpy(), o_ref, S_ref, TOL[dtype], f"segments {dtype} d={d}")


@pytest.mark.parametrize("dtype,d,H,lens", [("bf16", 64, 8, [512 * 64 + 21]),
                                            ("f32", 64, 4, [30000, 0, 37, 5000]),
                                            ("bf16", 32, 8, [20000, 1, 0, 14000])])
def test_long_packed_segment_schedule(g, dtype, d, H, lens):
    """Packed input of at most 32 (sequence, head) units averaging 128
    chunks or more: the segment bounds come from cu_seqlens on the device
    (G segments per sequence; short sequences leave empty segments, an empty
    sequence only empty ones).  Checked against the oracle."""
    cu = gi.cu_seqlens_from(lens)
    T = int(cu[-1])
    inp = gi.make_chunk_inputs(1, T, H, d, d, dtype, seed=47 + d, s0="normal", num_seqs=len(lens),
                               alpha_mean=8.0)
    print(f"case packed segment schedule {dtype} d={d} H={H} lens={lens}", flush=True)
    o, Sf = gpu_fwd(g, inp, 64, cu=cu)
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"], cu_seqlens=cu)
    check(o, Sf, o_ref, S_ref, TOL[dtype], f"packed segments {dtype} d={d}")


def test_long_sequence_segment_schedule_chunk16_no_states(g):
    """The segment schedule with chunk 16 (3000 tokens = 188 chunks, G = 8),
    no initial state and no final state wanted."""
    B, T, H, d, C = 1, 3000, 2, 32, 16
    inp = gi.make_chunk_inputs(B, T, H, d, d, "f32", seed=53, s0=None, alpha_mean=8.0)
    print(f"case segment schedule chunk 16 T={T}", flush=True)
    dd = to_dev(inp)
    o, Sf = g.chunk_fwd(*(dd[n] for n in NAMES), chunk=C, want_final=False)
    torch.cuda.synchronize()
    assert Sf is None
    o_ref, _ = oracle.fwd(*(inp[n] for n in NAMES))
    e = rel_err(o.cpu().numpy(), o_ref)
    print(f"segments chunk 16 err_o={e:.3e}", flush=True)
    assert e <= TOL["f32"]


def test_long_sequence_small_workspace_runs_the_serial_scan(g):
    """With a workspace sized for the plain two-pass path only, the default
    path runs it: the result equals the forced two-pass call bit for bit."""
    T, H, d, C = 512 * 64, 2, 64, 64
    inp = gi.make_chunk_inputs(1, T, H, d, d, "bf16", seed=43, s0="normal")
    print(f"case small workspace T={T}", flush=True)
    dd = to_dev(inp)
    o_t, S_t = g.chunk_fwd(*(dd[n] for n in NAMES), S0=dd["S0"], chunk=C, path="two_pass")
    # the plain two-pass size: a table and nc + 1 chunk slots of H heads
    slot_h = (g.workspace_bytes(1, C, H, d, d, 0, C, torch.bfloat16) - 256) // 2
    ws_small = 256 + (T // C + 1) * slot_h
    assert ws_small < g.workspace_bytes(1, T, H, d, d, 0, C, torch.bfloat16)
    ws = torch.empty(ws_small, dtype=torch.uint8, device="cuda")
    o_a, S_a = g.chunk_fwd(*(dd[n] for n in NAMES), S0=dd["S0"], chunk=C, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_t)
    assert torch.equal(S_a, S_t)


# ------------------------------------------------------------- properties
def test_state_aliasing_and_split_resume(g):
    inp = gi.make_chunk_inputs(2, 192, 2, 64, 64, "f32", seed=11, s0="normal")
    d = to_dev(inp)
    o_full, S_full = g.chunk_fwd(*(d[n] for n in NAMES), S0=d["S0"])
    T1 = 80
    first = {n: d[n][:, :T1].contiguous() for n in NAMES}
    second = {n: d[n][:, T1:].contiguous() for n in NAMES}
    S = d["S0"].clone()
    o1, _ = g.chunk_fwd(*(first[n] for n in NAMES), S0=S, S_final=S)  # in place
    o2, _ = g.chunk_fwd(*(second[n] for n in NAMES), S0=S, S_final=S)
    torch.cuda.synchronize()
    assert rel_err(torch.cat([o1, o2], 1).cpu().numpy(), o_full.cpu().numpy()) < 1e-5
    assert rel_err(S.cpu().numpy(), S_full.cpu().numpy()) < 1e-5


def test_zero_length_and_short(g):
    inp = gi.make_chunk_inputs(2, 0, 2, 16, 16, "f32", seed=12, s0="normal")
    d = to_dev(inp)
    o, Sf = g.chunk_fwd(*(d[n] for n in NAMES), S0=d["S0"], chunk=16)
    torch.cuda.synchronize()
    assert o.numel() == 0
    np.testing.assert_array_equal(Sf.cpu().numpy(), inp["S0"].numpy())
    o, Sf = g.chunk_fwd(*(d[n] for n in NAMES), chunk=16)
    torch.cuda.synchronize()
    assert float(Sf.abs().max()) == 0.0


def test_nan_propagates_within_unit(g):
    inp = gi.make_chunk_inputs(1, 96, 2, 64, 64, "f32", seed=13, s0="normal")
    inp["v"][0, 50, 1, 3] = float("nan")
    o, Sf = gpu_fwd(g, inp, 64)
    assert np.isfinite(o[0, :, 0]).all() and np.isfinite(Sf[0, 0]).all()  # other head clean
    assert np.isfinite(o[0, :48, 1]).all()                              # earlier chunk clean
    assert np.isnan(o[0, 50:, 1]).any() and np.isnan(Sf[0, 1]).any()


@pytest.mark.parametrize("path", ["two_pass", "fused"])
def test_deterministic(g, path):
    c, inp = make("small_2x512x4_d64")
    o1, S1 = gpu_fwd(g, inp, 64, path=path)
    o2, S2 = gpu_fwd(g, inp, 64, path=path)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(S1, S2)


def test_paths_agree_on_headline_shape(g):
    """Fused and two-pass kernels on one (batch) slice of the headline shape:
    both within tolerance of each other (they round intermediates at different
    points, so they are not bitwise equal)."""
    inp = gi.make_chunk_inputs(2, 1024, 16, 128, 128, "bf16", seed=77, s0="normal")
    o1, S1 = gpu_fwd(g, inp, 64, path="fused")
    o2, S2 = gpu_fwd(g, inp, 64, path="two_pass")
    assert rel_err(o1, o2) < 1e-2 and rel_err(S1, S2) < 1e-2


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("f32", 16)])
def test_decode_small(g, dtype, d):
    dd = gi.make_decode_inputs(5, 3, d, d, dtype, seed=40 + d, steps=6)
    S_gpu = dd["S"].cuda()
    S_ref = dd["S"].double().numpy()
    tol = TOL[dtype]
    for t in range(6):
        step = {n: dd[n][t].contiguous() for n in NAMES}
        o = g.decode_step(*(step[n].cuda() for n in NAMES), S_gpu)
        o_ref, S_ref = oracle.decode(*(step[n] for n in NAMES), S_ref)
        torch.cuda.synchronize()
        check(o.float().cpu().numpy(), S_gpu.cpu().numpy(), o_ref, S_ref, tol, f"decode {dtype} d={d} t={t}")


def test_decode_256x16_16_steps(g):
    c = gi.WORKLOADS["decode_256x16_d128"]
    dd = gi.make_decode_inputs(c["N"], c["H"], c["dk"], c["dv"], "bf16", c["seed"], steps=c["steps"])
    S_gpu = dd["S"].cuda()
    S_ref = dd["S"].double().numpy()
    dev = {n: dd[n].cuda() for n in NAMES}
    outs = []
    for t in range(c["steps"]):
        outs.append(g.decode_step(*(dev[n][t] for n in NAMES), S_gpu))
    torch.cuda.synchronize()
    for t in range(c["steps"]):
        o_ref, S_ref = oracle.decode(*(dd[n][t] for n in NAMES), S_ref)
        eo = rel_err(outs[t].float().cpu().numpy(), o_ref)
        assert eo <= TOL["bf16"], f"step {t}: o error {eo:.3e}"
    es = rel_err(S_gpu.cpu().numpy(), S_ref)
    print(f"decode 16 steps err_S={es:.3e}", flush=True)
    assert es <= TOL["bf16"]


def test_decode_streamed_equals_cached(g):
    """A state of 64 MiB or more is stepped with nontemporal loads and
    stores, a smaller one through the caches: the 256 x 16 heads state
    (256 MiB) in one call and the same sequences in calls of 32 (32 MiB
    each) give the same outputs and states, bit for bit."""
    c = gi.WORKLOADS["decode_256x16_d128"]
    dd = gi.make_decode_inputs(c["N"], c["H"], c["dk"], c["dv"], "bf16", c["seed"] + 1, steps=3)
    dev = {n: dd[n].cuda() for n in NAMES}
    S_all, S_part = dd["S"].cuda(), dd["S"].cuda()
    print("case decode streamed against cached", flush=True)
    for t in range(3):
        o_all = g.decode_step(*(dev[n][t] for n in NAMES), S_all)
        o_part = torch.empty_like(o_all)
        for n0 in range(0, c["N"], 32):
            g.decode_step(*(dev[n][t][n0:n0 + 32] for n in NAMES), S_part[n0:n0 + 32], out=o_part[n0:n0 + 32])
        torch.cuda.synchronize()
        assert torch.equal(o_all, o_part), f"step {t}: outputs differ"
    assert torch.equal(S_all, S_part)


def test_decode_steps_equal_chunk_forward(g):
    """T decode steps on the GPU agree with one chunked forward on the GPU."""
    dd = gi.make_decode_inputs(2, 2, 64, 64, "f32", seed=50, steps=40)
    S = dd["S"].cuda()
    outs = [g.decode_step(*(dd[n][t].cuda() for n in NAMES), S) for t in range(40)]
    seq = {n: dd[n].permute(1, 0, 2, 3).contiguous().cuda() for n in NAMES}
    o, Sf = g.chunk_fwd(*(seq[n] for n in NAMES), S0=dd["S"].cuda(), chunk=16)
    torch.cuda.synchronize()
    assert rel_err(torch.stack(outs, 1).cpu().numpy(), o.cpu().numpy()) < 1e-4
    assert rel_err(S.cpu().numpy(), Sf.cpu().numpy()) < 1e-4


# -------------------------------------------------------------- rule R1
@pytest.mark.parametrize("dtype,d,T", [("f32", 64, 150), ("bf16", 128, 200)])
def test_rule_r1_recurrent(g, dtype, d, T):
    """The alternative reading R1 on the token-by-token kernel against the
    oracle's R1, fixed-length with S0 and packed with an empty sequence."""
    inp = gi.make_chunk_inputs(2, T, 2, d, d, dtype, seed=31 + d, s0="normal")
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"], rule="R1")
    d_ = to_dev(inp)
    o, Sf = g.chunk_fwd(*(d_[n] for n in NAMES), S0=d_["S0"], recurrent=True, rule="R1")
    torch.cuda.synchronize()
    check(o.float().cpu().numpy(), Sf.cpu().numpy(), o_ref, S_ref, TOL[dtype], f"R1 {dtype} d={d}")
    # R1 and R5 differ for generic gates
    o5, _ = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"], rule="R5")
    assert rel_err(o5, o_ref) > 2 * TOL[dtype]
    lens = [90, 0, T - 90]
    cu = gi.cu_seqlens_from(lens)
    pk = gi.make_chunk_inputs(1, T, 2, d, d, dtype, seed=32 + d, s0="normal", num_seqs=3)
    o_ref, S_ref = oracle.fwd(*(pk[n] for n in NAMES), S0=pk["S0"], cu_seqlens=cu, rule="R1")
    d_ = to_dev(pk)
    o, Sf = g.chunk_fwd(*(d_[n] for n in NAMES), S0=d_["S0"], cu_seqlens=cu.cuda(), recurrent=True, rule="R1")
    torch.cuda.synchronize()
    check(o.float().cpu().numpy(), Sf.cpu().numpy(), o_ref, S_ref, TOL[dtype], f"R1 packed {dtype}")


def test_rule_r1_equals_r5_when_gates_collapse(g):
    """With b = w = beta both readings are KDA: the GPU's R1 and R5 agree."""
    inp = gi.make_chunk_inputs(1, 130, 2, 64, 64, "f32", seed=33, s0="normal", scalar_beta=True)
    d_ = to_dev(inp)
    o1, S1 = g.chunk_fwd(*(d_[n] for n in NAMES), S0=d_["S0"], recurrent=True, rule="R1")
    o5, S5 = g.chunk_fwd(*(d_[n] for n in NAMES), S0=d_["S0"], recurrent=True, rule="R5")
    torch.cuda.synchronize()
    assert rel_err(o1.cpu().numpy(), o5.cpu().numpy()) < 1e-5
    assert rel_err(S1.cpu().numpy(), S5.cpu().numpy()) < 1e-5


def test_rule_r1_rejected_on_single_pass_path(g):
    inp = to_dev(gi.make_chunk_inputs(1, 64, 1, 32, 32, "f32", seed=34))
    with pytest.raises(g.Gdn2Error) as e:
        g.chunk_fwd(*(inp[n] for n in NAMES), path="fused", rule="R1")
    assert e.value.status == 2


def gpu_fwd_r1(g, inp, chunk, cu=None, path="auto", layer_prep=False):
    d = to_dev(inp)
    o, Sf = g.chunk_fwd(*(d[n] for n in NAMES), S0=d.get("S0"), cu_seqlens=None if cu is None else cu.cuda(),
                        chunk=chunk, path=path, rule="R1", layer_prep=layer_prep)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), Sf.cpu().numpy()


# Rule R1 on the chunked two-pass path (its own per-chunk kernel; the state
# scan's R1 mode for bf16 with d = 32, 64, 128 and chunk 64, at one (6 and
# 10 units), two (48 units, d = 128) or, in the layer test, four column
# tiles per workgroup; the one-wave-per-tile R1 scan otherwise)
R1_CASES = [("f32", 16, 16, 1, 64, 1), ("f32", 64, 64, 2, 512, 4), ("f32", 128, 16, 2, 40, 2),
            ("f32", 32, 64, 2, 130, 3), ("bf16", 128, 64, 2, 200, 3), ("bf16", 64, 16, 2, 77, 3),
            ("bf16", 16, 64, 1, 90, 2), ("bf16", 128, 64, 4, 300, 12), ("bf16", 64, 64, 2, 333, 5),
            ("bf16", 32, 64, 3, 150, 2)]


@pytest.mark.parametrize("path", ["auto", "two_pass"])
@pytest.mark.parametrize("dtype,d,chunk,B,T,H", R1_CASES)
def test_rule_r1_chunked(g, dtype, d, chunk, B, T, H, path):
    inp = gi.make_chunk_inputs(B, T, H, d, d, dtype, seed=120 + d + T, s0="normal")
    print(f"case R1 chunked {dtype} d={d} C={chunk} B={B} T={T} H={H} {path}", flush=True)
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"], rule="R1")
    o, Sf = gpu_fwd_r1(g, inp, chunk, path=path)
    check(o, Sf, o_ref, S_ref, TOL[dtype], f"R1 chunked {dtype} d={d} C={chunk} {path}")


def test_rule_r1_chunked_packed_and_extreme_decay(g):
    """Packed input with empty and one-token sequences; then decays down to
    1e-4 and zero (the pairwise diagonal blocks of both product families)."""
    lens = [70, 0, 1, 64, 130, 0, 15]
    cu = gi.cu_seqlens_from(lens)
    inp = gi.make_chunk_inputs(1, int(cu[-1]), 2, 64, 64, "f32", seed=131, s0="normal", num_seqs=len(lens))
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"], cu_seqlens=cu, rule="R1")
    for chunk in (16, 64):
        print(f"case R1 packed C={chunk}", flush=True)
        o, Sf = gpu_fwd_r1(g, inp, chunk, cu=cu)
        check(o, Sf, o_ref, S_ref, TOL["f32"], f"R1 packed C={chunk}")
    # bf16, d = 128: the scan's R1 mode on packed sequences with ragged ends
    inp = gi.make_chunk_inputs(1, int(cu[-1]), 3, 128, 128, "bf16", seed=135, s0="normal", num_seqs=len(lens))
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"], cu_seqlens=cu, rule="R1")
    print("case R1 packed bf16 d=128 C=64", flush=True)
    o, Sf = gpu_fwd_r1(g, inp, 64, cu=cu)
    check(o, Sf, o_ref, S_ref, TOL["bf16"], "R1 packed bf16 d=128 C=64")
    for dtype, d, chunk in (("f32", 64, 64), ("bf16", 128, 64), ("f32", 32, 16)):
        inp = gi.make_strong_decay_inputs(2, 150, 2, d, d, dtype, seed=132 + d, s0="normal")
        print(f"case R1 strong decay {dtype} d={d} C={chunk}", flush=True)
        o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"], rule="R1")
        o, Sf = gpu_fwd_r1(g, inp, chunk)
        check(o, Sf, o_ref, S_ref, TOL[dtype], f"R1 strong decay {dtype} d={d} C={chunk}")


def test_rule_r1_chunked_gate_layouts(g):
    """Per-(token, head) gates (b = w = beta: both readings are KDA, so R1
    equals R5) and layer prep, against the oracle."""
    from oracle import layer_prep as lp
    inp = gi.make_chunk_inputs(2, 190, 3, 64, 64, "f32", seed=133, s0="normal", scalar_beta=True)
    compact = dict(inp, b=inp["b"][..., 0].contiguous(), w=inp["w"][..., 0].contiguous())
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"], rule="R1")
    print("case R1 KDA gates", flush=True)
    o, Sf = gpu_fwd_r1(g, compact, 64)
    check(o, Sf, o_ref, S_ref, TOL["f32"], "R1 KDA gates")
    raw = gi.make_layer_inputs(2, 200, 3, 128, 128, "bf16", seed=134, s0="normal")
    prep = lp.layer_prep(raw["q"], raw["k"], raw["alpha"], raw["b"], raw["w"])
    o_ref, S_ref = oracle.fwd(prep["q"], prep["k"], raw["v"], prep["alpha"], prep["b"], prep["w"], S0=raw["S0"],
                              rule="R1")
    print("case R1 layer prep", flush=True)
    o, Sf = gpu_fwd_r1(g, raw, 64, layer_prep=True)
    check(o, Sf, o_ref, S_ref, TOL["bf16"], "R1 layer prep")


def test_rule_r1_chunked_layer_8x4096x16(g):
    """Rule R1 on the layer workload (B=8, T=4096, H=16, d=128, bf16): every
    element against the oracle's R1."""
    c, inp = make("layer_8x4096x16_d128")
    print("case R1 layer 8x4096x16", flush=True)
    o, Sf = gpu_fwd_r1(g, inp, 64)
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), rule="R1")
    check(o, Sf, o_ref, S_ref, TOL["bf16"], "R1 layer")


def test_binding_rejects_wrong_tensors(g):
    """The binding checks every tensor's shape, dtype, device and layout
    before it calls the library (no launch happens for these)."""
    inp = to_dev(gi.make_chunk_inputs(2, 64, 2, 32, 32, "bf16", seed=90))
    args = [inp[n] for n in NAMES]
    bad = [
        dict(k=inp["k"][:, :32].contiguous()),                       # k shorter than q
        dict(v=inp["v"].float()),                                    # dtype
        dict(k=inp["k"].cpu()),                                      # device
        dict(v=inp["v"].transpose(0, 1)),                            # not contiguous
    ]
    for over in bad:
        a = [over.get(n, inp[n]) for n in NAMES]
        with pytest.raises((ValueError, TypeError)):
            g.chunk_fwd(*a, chunk=16)
    for kw in (dict(out=torch.empty((2, 64, 2, 16), dtype=torch.bfloat16, device="cuda")),
               dict(out=torch.empty((2, 64, 2, 32), dtype=torch.float32, device="cuda")),
               dict(S_final=torch.empty((2, 2, 32, 32), dtype=torch.bfloat16, device="cuda")),
               dict(S_final=torch.empty((3, 2, 32, 32), dtype=torch.float32, device="cuda")),
               dict(workspace=torch.empty(64, dtype=torch.uint8))):
        with pytest.raises((ValueError, TypeError)):
            g.chunk_fwd(*args, chunk=16, **kw)
    d = gi.make_decode_inputs(4, 2, 32, 32, "bf16", seed=91, steps=1)
    dd = {n: d[n][0].cuda() for n in NAMES}
    S = d["S"].cuda()
    for name, t in (("k", dd["k"][:3].contiguous()), ("w", dd["w"].float()), ("alpha", dd["alpha"][..., :16].contiguous())):
        a = [t if n == name else dd[n] for n in NAMES]
        with pytest.raises((ValueError, TypeError)):
            g.decode_step(*a, S)
    with pytest.raises((ValueError, TypeError)):
        g.decode_step(*(dd[n] for n in NAMES), S, out=torch.empty((4, 2, 16), dtype=torch.bfloat16, device="cuda"))
