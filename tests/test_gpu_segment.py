"""GPU parity of the segment state maps (gdn2_chunk_segment_map) and of their
exclusive scan (gdn2_segment_combine) against the float64 oracle (MI355X
only).  Maps and states are compared element by element: max |x - ref| /
max |ref| <= 1e-4 for float32 inputs and 2e-2 for bfloat16 inputs (the
forward's bars).  The end-to-end case cuts one long sequence into segments,
chains their maps and runs every segment from its entering state: the
outputs must be those of the whole sequence."""
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


def gpu_map(g, inp, chunk, cu=None, layer_prep=False):
    d = {n: inp[n].cuda() for n in NAMES}
    Phi, Psi = g.segment_map(*(d[n] for n in NAMES), cu_seqlens=None if cu is None else cu.cuda(),
                             chunk=chunk, layer_prep=layer_prep)
    torch.cuda.synchronize()
    return Phi.cpu().numpy(), Psi.cpu().numpy()


def check_map(got, ref, tol, label):
    for name, x, r in (("Phi", got[0], ref[0]), ("Psi", got[1], ref[1])):
        e = rel_err(x, r)
        print(f"{label} {name} err={e:.3e}", flush=True)
        assert e <= tol, f"{label}: {name} error {e:.3e} > {tol}"


CASES = [  # dtype, d, chunk, B, T, H
    ("f32", 16, 16, 2, 77, 2),
    ("f32", 32, 64, 1, 190, 2),
    ("f32", 64, 64, 2, 130, 1),
    ("f32", 128, 16, 1, 100, 1),
    ("f32", 128, 64, 1, 150, 1),
    ("bf16", 64, 16, 2, 77, 2),
    ("bf16", 128, 64, 2, 300, 2),
    ("bf16", 16, 64, 1, 64, 3),
    ("bf16", 16, 16, 2, 50, 2),
    ("bf16", 32, 64, 1, 130, 2),
]


@pytest.mark.parametrize("dtype,d,chunk,B,T,H", CASES)
def test_segment_map_small(g, dtype, d, chunk, B, T, H):
    inp = gi.make_chunk_inputs(B, T, H, d, d, dtype, seed=600 + d + T, alpha_mean=6.0)
    print(f"case map {dtype} d={d} C={chunk} B={B} T={T} H={H}", flush=True)
    got = gpu_map(g, inp, chunk)
    ref = oracle.segment_map(*(inp[n] for n in NAMES))
    check_map(got, ref, TOL[dtype], f"map {dtype} d={d} C={chunk} T={T}")


def test_segment_map_packed_with_empty_segments(g):
    lens = [70, 0, 1, 64, 130, 0, 15]
    cu = gi.cu_seqlens_from(lens)
    T = int(cu[-1])
    inp = gi.make_chunk_inputs(1, T, 2, 64, 64, "f32", seed=31, num_seqs=len(lens), alpha_mean=6.0)
    ref = oracle.segment_map(*(inp[n] for n in NAMES), cu_seqlens=cu)
    for chunk in (16, 64):
        print(f"case map packed C={chunk}", flush=True)
        got = gpu_map(g, inp, chunk, cu=cu)
        check_map(got, ref, TOL["f32"], f"map packed C={chunk}")
        for i in (1, 5):  # empty segments: Phi = I, Psi = 0 exactly
            np.testing.assert_array_equal(got[0][i], np.broadcast_to(np.eye(64), (2, 64, 64)))
            np.testing.assert_array_equal(got[1][i], 0.0)


def test_segment_map_zero_length(g):
    inp = gi.make_chunk_inputs(2, 0, 2, 32, 32, "f32", seed=3)
    print("case map T=0", flush=True)
    Phi, Psi = gpu_map(g, inp, 64)
    np.testing.assert_array_equal(Phi, np.broadcast_to(np.eye(32), (2, 2, 32, 32)))
    np.testing.assert_array_equal(Psi, 0.0)


@pytest.mark.parametrize("case", ["kda", "gdn", "layer_prep"])
def test_segment_map_gate_modes(g, case):
    d, T = 128, 200
    if case == "layer_prep":
        from oracle import layer_prep as lp
        raw = gi.make_layer_inputs(1, T, 2, d, d, "bf16", seed=640, scalar_beta=True)
        prep = lp.layer_prep(raw["q"], raw["k"], raw["alpha"], raw["b"], raw["w"])
        full = {x: (prep[x][..., None] * np.ones(d) if prep[x].ndim == 3 else prep[x])
                for x in ("q", "k", "alpha", "b", "w")}
        full["v"] = raw["v"]
        print("case map layer prep", flush=True)
        got = gpu_map(g, raw, 64, layer_prep=True)
    else:
        inp = gi.make_chunk_inputs(1, T, 2, d, d, "bf16", seed=641, scalar_beta=True, alpha_mean=6.0)
        full, compact = dict(inp), dict(inp)
        for x in (("b", "w") if case == "kda" else ("b", "w", "alpha")):
            s = inp[x][..., 0].contiguous()
            compact[x] = s
            full[x] = s[..., None].expand_as(inp[x]).contiguous()
        print(f"case map {case}", flush=True)
        got = gpu_map(g, compact, 64)
    ref = oracle.segment_map(*(full[n] for n in NAMES))
    check_map(got, ref, TOL["bf16"], f"map {case}")


@pytest.mark.parametrize("d,G,H", [(16, 5, 3), (64, 4, 2), (128, 6, 2), (128, 8, 3), (32, 16, 2), (64, 2, 5),
                                   (16, 1, 2)])
def test_segment_combine(g, d, G, H):
    rng = np.random.default_rng(700 + d)
    # maps of the size real segments give: Phi contracts, Psi of order one
    Phi = (0.9 * np.eye(d) + rng.normal(0.0, 0.3 / np.sqrt(d), (G, H, d, d))).astype(np.float32)
    Psi = rng.standard_normal((G, H, d, d)).astype(np.float32)
    S0 = rng.normal(0.0, 0.1, (H, d, d)).astype(np.float32)
    for s0 in (None, S0):
        print(f"case combine d={d} G={G} S0={'yes' if s0 is not None else 'no'}", flush=True)
        S_in, Sf = g.segment_combine(torch.from_numpy(Phi).cuda(), torch.from_numpy(Psi).cuda(),
                                     None if s0 is None else torch.from_numpy(s0).cuda())
        torch.cuda.synchronize()
        ref_in, ref_f = oracle.segment_combine(Phi, Psi, s0)
        e = max(rel_err(S_in.cpu().numpy(), ref_in), rel_err(Sf.cpu().numpy(), ref_f))
        print(f"combine d={d} err={e:.3e}", flush=True)
        assert e <= TOL["f32"]
        if s0 is not None:
            np.testing.assert_array_equal(S_in[0].cpu().numpy(), s0)


def test_segment_combine_no_segments(g):
    S0 = torch.randn(2, 32, 32).cuda()
    print("case combine G=0", flush=True)
    S_in, Sf = g.segment_combine(torch.empty(0, 2, 32, 32).cuda(), torch.empty(0, 2, 32, 32).cuda(), S0)
    torch.cuda.synchronize()
    assert S_in.shape == (0, 2, 32, 32)
    assert torch.equal(Sf, S0)


def run_segmented(g, inp, lens, chunk, S0=None):
    """Maps of every segment, their scan from S0, then every segment from
    its entering state, all on the GPU.  Returns (o, S_in, S_final of the
    scan, S_final of every segment's run, Phi, Psi)."""
    cu = gi.cu_seqlens_from(lens).cuda()
    d = {n: inp[n].cuda() for n in NAMES}
    Phi, Psi = g.segment_map(*(d[n] for n in NAMES), cu_seqlens=cu, chunk=chunk)
    S_in, Sf = g.segment_combine(Phi, Psi, None if S0 is None else S0.cuda())
    o, Sf_seg = g.chunk_fwd(*(d[n] for n in NAMES), S0=S_in, cu_seqlens=cu, chunk=chunk)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy(), S_in.cpu().numpy(), Sf.cpu().numpy(), Sf_seg.cpu().numpy(),
            Phi.cpu().numpy(), Psi.cpu().numpy())


@pytest.mark.parametrize("dtype,d,chunk,lens", [
    ("f32", 64, 64, [250, 0, 333, 64, 353]),
    ("f32", 32, 16, [100, 100, 1, 99]),
    ("bf16", 128, 64, [512, 300, 700, 8]),
])
def test_segments_reproduce_the_sequence(g, dtype, d, chunk, lens):
    T, H = sum(lens), 2
    inp = gi.make_chunk_inputs(1, T, H, d, d, dtype, seed=800 + T, s0="normal", alpha_mean=8.0)
    print(f"case segmented {dtype} d={d} C={chunk} lens={lens}", flush=True)
    o, S_in, Sf, Sf_seg, _, _ = run_segmented(g, inp, lens, chunk, S0=inp["S0"][0])
    o_ref, Sf_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    e_o, e_f, e_l = rel_err(o, o_ref), rel_err(Sf, Sf_ref[0]), rel_err(Sf_seg[-1], Sf_ref[0])
    print(f"segmented {dtype} d={d} o err={e_o:.3e} S_final err={e_f:.3e} last segment {e_l:.3e}", flush=True)
    assert max(e_o, e_f, e_l) <= TOL[dtype]


@pytest.mark.parametrize("dtype,d,chunk,lens", [
    ("f32", 64, 64, [250, 0, 333, 64, 353]),
    ("bf16", 128, 64, [512, 300, 700, 8]),
    ("bf16", 32, 16, [100, 1, 99]),
])
def test_prepared_rerun_equals_full_rerun(g, dtype, d, chunk, lens):
    """gdn2_chunk_fwd with GDN2_FLAG_PREPARED on the workspace that the
    segment maps left runs the state scan alone; outputs and final states
    equal those of the full forward from the same entering states bit for
    bit (the same per-chunk kernel wrote the workspace)."""
    T, H = sum(lens), 2
    inp = gi.make_chunk_inputs(1, T, H, d, d, dtype, seed=900 + T, s0="normal", alpha_mean=8.0)
    print(f"case prepared rerun {dtype} d={d} C={chunk} lens={lens}", flush=True)
    cu = gi.cu_seqlens_from(lens).cuda()
    dd = {n: inp[n].cuda() for n in NAMES}
    ws = torch.empty(g.workspace_bytes(1, T, H, d, d, len(lens), chunk, dd["q"].dtype), dtype=torch.uint8,
                     device="cuda")
    Phi, Psi = g.segment_map(*(dd[n] for n in NAMES), cu_seqlens=cu, chunk=chunk, workspace=ws)
    S_in, _ = g.segment_combine(Phi, Psi, inp["S0"][0].cuda())
    o_p, Sf_p = g.chunk_fwd(*(dd[n] for n in NAMES), S0=S_in, cu_seqlens=cu, chunk=chunk, workspace=ws,
                            prepared=True)
    o_f, Sf_f = g.chunk_fwd(*(dd[n] for n in NAMES), S0=S_in, cu_seqlens=cu, chunk=chunk, path="two_pass")
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_f)
    assert torch.equal(Sf_p, Sf_f)


def test_prepared_workspace_of_a_forward_call(g):
    """A workspace filled by a two-pass forward serves a prepared call from
    another initial state (fixed-length batch, ragged last chunk)."""
    B, T, H, d, C = 3, 200, 2, 64, 64
    inp = gi.make_chunk_inputs(B, T, H, d, d, "bf16", seed=77, s0="normal")
    print(f"case prepared forward workspace B={B} T={T}", flush=True)
    dd = {n: inp[n].cuda() for n in NAMES}
    ws = torch.empty(g.workspace_bytes(B, T, H, d, d, 0, C, torch.bfloat16), dtype=torch.uint8, device="cuda")
    g.chunk_fwd(*(dd[n] for n in NAMES), chunk=C, workspace=ws, path="two_pass")
    S1 = inp["S0"].cuda()
    o_p, Sf_p = g.chunk_fwd(*(dd[n] for n in NAMES), S0=S1, chunk=C, workspace=ws, prepared=True)
    o_f, Sf_f = g.chunk_fwd(*(dd[n] for n in NAMES), S0=S1, chunk=C, path="two_pass")
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_f)
    assert torch.equal(Sf_p, Sf_f)


def test_segments_per_rank_shape(g):
    """The packed workload's 32768-token stream (H=16, d=128, bf16) as one sequence cut
    into 8 segments of 4096 tokens, the per-rank share of an 8-way
    context-parallel split, with long-memory decay so the state crosses
    every boundary.  The oracle recomputes two heads end to end: their
    maps of one segment, every entering state, and all outputs."""
    H, d, G, L = 16, 128, 8, 4096
    inp = gi.make_chunk_inputs(1, G * L, H, d, d, "bf16", seed=3, alpha_mean=8.0)
    print("case segmented per-rank shape", flush=True)
    o, S_in, Sf, _, Phi, Psi = run_segmented(g, inp, [L] * G, 64)
    assert np.isfinite(o).all() and np.isfinite(S_in).all()
    cu = gi.cu_seqlens_from([L] * G)
    for hh in (0, 11):
        sub = {x: inp[x][:, :, hh:hh + 1].contiguous() for x in NAMES}
        Phi_r, Psi_r = oracle.segment_map(*(sub[x] for x in NAMES), cu_seqlens=cu)
        S_in_r, Sf_r = oracle.segment_combine(Phi_r, Psi_r)
        o_r, _ = oracle.fwd(*(sub[x] for x in NAMES))
        gs = 5 if hh == 0 else 2
        errs = (rel_err(Phi[gs, hh], Phi_r[gs, 0]), rel_err(Psi[gs, hh], Psi_r[gs, 0]),
                rel_err(S_in[:, hh], S_in_r[:, 0]), rel_err(Sf[hh], Sf_r[0]), rel_err(o[:, :, hh], o_r[:, :, 0]))
        print(f"per-rank h={hh} Phi err={errs[0]:.3e} Psi err={errs[1]:.3e} S_in err={errs[2]:.3e} "
              f"S_final err={errs[3]:.3e} o err={errs[4]:.3e}", flush=True)
        assert max(errs) <= TOL["bf16"]
