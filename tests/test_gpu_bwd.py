"""GPU parity of the chunked backward (gdn2_chunk_bwd) against the float64
oracle backward (MI355X only).  Every gradient tensor is compared element by
element: max |x - ref| / max |ref| <= 1e-4 for float32 inputs and 2e-2 for
bfloat16 inputs (the forward's bars), on the same stored inputs and incoming
gradients."""
import numpy as np
import pytest
import torch

import gdn2_inputs as gi
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("q", "k", "v", "alpha", "b", "w")
GRADS = ("dq", "dk", "dv", "dalpha", "db", "dw")


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


def gpu_bwd(g, inp, grads, chunk, cu=None):
    d = {n: inp[n].cuda() for n in NAMES}
    S0 = inp.get("S0")
    dSf = grads["dS_final"]
    out = g.chunk_bwd(*(d[n] for n in NAMES), grads["dout"].cuda(),
                      S0=None if S0 is None else S0.cuda(), dS_final=None if dSf is None else dSf.cuda(),
                      cu_seqlens=None if cu is None else cu.cuda(), chunk=chunk)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() for k, v in out.items() if v is not None}


def check(got, ref, tol, label, sel=None):
    for name in GRADS + ("dS0",):
        x = got[name] if sel is None else sel(name, got[name])
        e = rel_err(x, ref[name])
        print(f"{label} {name} err={e:.3e}", flush=True)
        assert e <= tol, f"{label}: {name} error {e:.3e} > {tol}"


CASES = [  # dtype, d, chunk, B, T, H, s0, dS_final
    ("f32", 32, 16, 2, 77, 2, "normal", True),
    ("f32", 64, 64, 1, 190, 2, "normal", True),
    ("f32", 128, 64, 1, 130, 1, None, False),
    ("f32", 16, 64, 2, 64, 1, None, True),
    ("bf16", 128, 64, 1, 200, 2, "normal", True),
    ("bf16", 16, 64, 2, 100, 1, None, True),
    ("bf16", 64, 16, 1, 77, 2, "normal", False),
]


@pytest.mark.parametrize("dtype,d,chunk,B,T,H,s0,with_dS", CASES)
def test_bwd_small(g, dtype, d, chunk, B, T, H, s0, with_dS):
    seed = 100 + d + T
    inp = gi.make_chunk_inputs(B, T, H, d, d, dtype, seed, s0=s0)
    grads = gi.make_bwd_grads(B, T, H, d, d, dtype, seed, with_dS=with_dS)
    print(f"case {dtype} d={d} C={chunk} B={B} T={T} H={H}", flush=True)
    got = gpu_bwd(g, inp, grads, chunk)
    ref = oracle.bwd(*(inp[n] for n in NAMES), grads["dout"], S0=inp["S0"], dS_final=grads["dS_final"])
    check(got, ref, TOL[dtype], f"{dtype} d={d} C={chunk} T={T}")


def test_bwd_packed_with_empty_sequences(g):
    lens = [70, 0, 1, 64, 130, 0, 15]
    cu = gi.cu_seqlens_from(lens)
    T = int(cu[-1])
    inp = gi.make_chunk_inputs(1, T, 2, 64, 64, "f32", seed=19, s0="normal", num_seqs=len(lens))
    grads = gi.make_bwd_grads(1, T, 2, 64, 64, "f32", seed=19, num_seqs=len(lens))
    ref = oracle.bwd(*(inp[n] for n in NAMES), grads["dout"], S0=inp["S0"], dS_final=grads["dS_final"],
                     cu_seqlens=cu)
    for chunk in (16, 64):
        print(f"case packed C={chunk}", flush=True)
        got = gpu_bwd(g, inp, grads, chunk, cu=cu)
        check(got, ref, TOL["f32"], f"packed C={chunk}")


def test_bwd_zero_length(g):
    inp = gi.make_chunk_inputs(2, 0, 2, 32, 32, "f32", seed=3, s0="normal")
    grads = gi.make_bwd_grads(2, 0, 2, 32, 32, "f32", seed=3)
    print("case T=0", flush=True)
    got = gpu_bwd(g, inp, grads, 64)
    np.testing.assert_array_equal(got["dS0"], grads["dS_final"].numpy())


@pytest.mark.parametrize("dtype,d,chunk,B,T,H,lens", [
    ("f32", 32, 64, 1, 130 * 64 + 5, 2, None),
    ("f32", 32, 16, 1, 3000, 2, None),
    ("bf16", 64, 64, 2, 140 * 64 - 7, 4, None),
    ("f32", 32, 64, 1, None, 4, [30000, 0, 37, 5000]),
    ("bf16", 32, 64, 2, 130 * 64 + 3, 16, None),
])
def test_bwd_segment_schedule(g, dtype, d, chunk, B, T, H, lens):
    """Sequences of 128 chunks or more with at most 32 (sequence, head)
    units: both scans of the backward take the segment schedule (the
    forward maps and their scan for the states; per-segment reverse scans
    from zero, the adjoint scan of the maps and the final reverse scans for
    the state gradients).  Every gradient, and dS0, against the oracle's;
    fixed-length and packed (empty and sub-chunk sequences), chunks 64 and
    16."""
    cu = None if lens is None else gi.cu_seqlens_from(lens)
    if cu is not None:
        T = int(cu[-1])
    n = None if lens is None else len(lens)
    inp = gi.make_chunk_inputs(B, T, H, d, d, dtype, seed=61 + d, s0="normal", num_seqs=n, alpha_mean=8.0)
    grads = gi.make_bwd_grads(B, T, H, d, d, dtype, seed=61 + d, num_seqs=n)
    print(f"case bwd segment schedule {dtype} d={d} C={chunk} B={B} T={T} H={H} lens={lens}", flush=True)
    got = gpu_bwd(g, inp, grads, chunk, cu=cu)
    ref = oracle.bwd(*(inp[x] for x in NAMES), grads["dout"], S0=inp["S0"], dS_final=grads["dS_final"],
                     cu_seqlens=cu)
    check(got, ref, TOL[dtype], f"bwd segments {dtype} d={d} C={chunk}")


def test_bwd_deterministic(g):
    inp = gi.make_chunk_inputs(1, 300, 2, 128, 128, "bf16", seed=21, s0="normal")
    grads = gi.make_bwd_grads(1, 300, 2, 128, 128, "bf16", seed=21)
    print("case deterministic", flush=True)
    a = gpu_bwd(g, inp, grads, 64)
    b = gpu_bwd(g, inp, grads, 64)
    for name in a:
        np.testing.assert_array_equal(a[name], b[name])


def test_bwd_layer_8x4096x16_all_units(g):
    """Full headline size (B=8, T=4096, H=16, d=128, bf16) with dL/dS_final:
    every element of every gradient and of dS0 against the oracle's backward
    of the whole layer (all 128 (batch, head) units)."""
    c = gi.WORKLOADS["layer_8x4096x16_d128"]
    inp = gi.make_chunk_inputs(c["B"], c["T"], c["H"], c["dk"], c["dv"], "bf16", c["seed"], s0=c["s0"])
    grads = gi.make_bwd_grads(c["B"], c["T"], c["H"], c["dk"], c["dv"], "bf16", c["seed"])
    print("case layer backward", flush=True)
    got = gpu_bwd(g, inp, grads, 64)
    ref = oracle.bwd(*(inp[x] for x in NAMES), grads["dout"], S0=inp["S0"], dS_final=grads["dS_final"])
    check(got, ref, TOL["bf16"], "layer backward")


def gpu_bwd_raw(g, inp, grads, chunk, layer_prep=False):
    d = {n: inp[n].cuda() for n in NAMES}
    S0 = inp.get("S0")
    dSf = grads["dS_final"]
    out = g.chunk_bwd(*(d[n] for n in NAMES), grads["dout"].cuda(),
                      S0=None if S0 is None else S0.cuda(), dS_final=None if dSf is None else dSf.cuda(),
                      chunk=chunk, layer_prep=layer_prep)
    torch.cuda.synchronize()
    for name, x in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dalpha", "alpha"), ("db", "b"), ("dw", "w")):
        assert tuple(out[name].shape) == tuple(inp[x].shape) and out[name].dtype == inp[x].dtype, name
    return {k: v.float().cpu().numpy() for k, v in out.items() if v is not None}


# Gates per (token, head): the GPU reads the compact [B, T, H] tensors; the
# oracle gets the same values repeated over the channels and its per-channel
# gradients are summed over them (oracle/layer_prep.py sum_to_layout).
GATE_CASES = {"kda": ("b", "w"), "gdn": ("b", "w", "alpha"), "b_only": ("b",), "w_only": ("w",)}


@pytest.mark.parametrize("dtype,d,T,chunk", [("f32", 64, 190, 64), ("bf16", 128, 200, 64), ("bf16", 32, 77, 16),
                                             ("f32", 32, 130 * 64, 64)])  # the last: segment schedule
@pytest.mark.parametrize("case", list(GATE_CASES))
def test_bwd_per_token_gates(g, case, dtype, d, T, chunk):
    from oracle import layer_prep as lp
    inp = gi.make_chunk_inputs(2, T, 3, d, d, dtype, seed=900 + T, s0="normal",
                               scalar_beta=(case in ("kda", "gdn")))
    grads = gi.make_bwd_grads(2, T, 3, d, d, dtype, seed=900 + T)
    full, compact = dict(inp), dict(inp)
    for x in GATE_CASES[case]:
        s = inp[x][..., 0].contiguous()
        compact[x] = s
        full[x] = s[..., None].expand_as(inp[x]).contiguous()
    print(f"case bwd gates {case} {dtype} d={d} C={chunk}", flush=True)
    got = gpu_bwd_raw(g, compact, grads, chunk)
    ref = oracle.bwd(*(full[n] for n in NAMES), grads["dout"], S0=inp["S0"], dS_final=grads["dS_final"])
    for name, x in (("db", "b"), ("dw", "w"), ("dalpha", "alpha")):
        ref[name] = lp.sum_to_layout(ref[name], compact[x].float().numpy())
    check(got, ref, TOL[dtype], f"bwd gates {case} {dtype} d={d}")


# Layer prep: raw q, k, gate logits and the float32 log-decay go in; the
# oracle prepares them in float64, takes the recurrence's gradients and
# carries them back through the prep (oracle/layer_prep.py layer_prep_bwd).
@pytest.mark.parametrize("dtype,d,T,chunk", [("f32", 64, 150, 64), ("bf16", 128, 200, 64), ("bf16", 64, 77, 16)])
@pytest.mark.parametrize("scalar", [False, True])
def test_bwd_layer_prep(g, dtype, d, T, chunk, scalar):
    from oracle import layer_prep as lp
    raw = gi.make_layer_inputs(2, T, 3, d, d, dtype, seed=950 + T, s0="normal", scalar_beta=scalar)
    grads = gi.make_bwd_grads(2, T, 3, d, d, dtype, seed=950 + T)
    prep = lp.layer_prep(raw["q"], raw["k"], raw["alpha"], raw["b"], raw["w"])
    full = {x: (prep[x][..., None] * np.ones(d) if prep[x].ndim == 3 else prep[x])
            for x in ("q", "k", "alpha", "b", "w")}
    print(f"case bwd layer prep {dtype} d={d} C={chunk} scalar={scalar}", flush=True)
    got = gpu_bwd_raw(g, raw, grads, chunk, layer_prep=True)
    gp = oracle.bwd(full["q"], full["k"], raw["v"], full["alpha"], full["b"], full["w"], grads["dout"],
                    S0=raw["S0"], dS_final=grads["dS_final"])
    ref = lp.layer_prep_bwd(raw["q"], raw["k"], raw["alpha"], raw["b"], raw["w"], gp)
    ref["dS0"] = gp["dS0"]
    check(got, ref, TOL[dtype], f"bwd layer prep {dtype} d={d} scalar={scalar}")


def test_bwd_rejects_path_and_rule_flags(g):
    inp = gi.make_chunk_inputs(1, 32, 1, 16, 16, "f32", seed=5)
    grads = gi.make_bwd_grads(1, 32, 1, 16, 16, "f32", seed=5)
    d = {n: inp[n].cuda() for n in NAMES}
    lib = g.lib()
    ws = torch.empty(g.bwd_workspace_bytes(1, 32, 1, 16, 16, 0, 16, torch.float32), dtype=torch.uint8, device="cuda")
    outs = [torch.empty_like(d[n]) for n in NAMES]
    for flag in (g.FLAG_RECURRENT, g.FLAG_FUSED, g.FLAG_RULE_R1):
        st = lib.gdn2_chunk_bwd(*(d[n].data_ptr() for n in NAMES), None, None, 1, 32, 1, 16, 16, 0, 16, 0, flag,
                                grads["dout"].cuda().data_ptr(), None, *(o.data_ptr() for o in outs), None,
                                ws.data_ptr(), ws.numel(), None)
        assert st == 2


RECT_CASES = [  # dtype, dk, dv, chunk, B, T, H, s0, dS_final
    ("f32", 16, 64, 16, 2, 77, 2, "normal", True),
    ("f32", 128, 32, 64, 1, 130, 2, "normal", True),
    ("bf16", 64, 128, 64, 2, 100, 2, None, True),
    ("bf16", 128, 16, 64, 1, 150, 2, "normal", False),
]


@pytest.mark.parametrize("dtype,dk,dv,chunk,B,T,H,s0,with_dS", RECT_CASES)
def test_bwd_rect_heads(g, dtype, dk, dv, chunk, B, T, H, s0, with_dS):
    """dk != dv: the square backward on max(dk, dv) over widened inputs,
    every gradient and dL/dS0 narrowed back, against the oracle."""
    seed = 140 + dk + 3 * dv + T
    inp = gi.make_chunk_inputs(B, T, H, dk, dv, dtype, seed, s0=s0)
    grads = gi.make_bwd_grads(B, T, H, dk, dv, dtype, seed, with_dS=with_dS)
    print(f"case rect {dtype} dk={dk} dv={dv} C={chunk} B={B} T={T} H={H}", flush=True)
    got = gpu_bwd(g, inp, grads, chunk)
    ref = oracle.bwd(*(inp[n] for n in NAMES), grads["dout"], S0=inp["S0"], dS_final=grads["dS_final"])
    for name in GRADS + ("dS0",):
        assert got[name].shape == np.asarray(ref[name]).shape, name
    check(got, ref, TOL[dtype], f"rect {dtype} {dk}x{dv} C={chunk}")


def test_bwd_rect_heads_gates_and_packed(g):
    """dk != dv with b, w and alpha per (token, head) (their gradients are
    [B, T, H], not widened) and with packed sequences."""
    from oracle import layer_prep as lp
    inp = gi.make_chunk_inputs(2, 120, 2, 64, 32, "f32", seed=151, s0="normal", scalar_beta=True)
    grads = gi.make_bwd_grads(2, 120, 2, 64, 32, "f32", 151, with_dS=True)
    full, compact = dict(inp), dict(inp)
    for x in ("b", "w", "alpha"):
        s = inp[x][..., 0].contiguous()
        compact[x] = s
        full[x] = s[..., None].expand_as(inp[x]).contiguous()
    print("case rect per-token gates", flush=True)
    got = gpu_bwd_raw(g, compact, grads, 64)
    ref = oracle.bwd(*(full[n] for n in NAMES), grads["dout"], S0=inp["S0"], dS_final=grads["dS_final"])
    for name, x in (("db", "b"), ("dw", "w"), ("dalpha", "alpha")):
        ref[name] = lp.sum_to_layout(ref[name], compact[x].float().numpy())
    check(got, ref, TOL["f32"], "rect per-token gates")
    lens = [70, 0, 1, 64, 130, 15]
    cu = gi.cu_seqlens_from(lens)
    inp = gi.make_chunk_inputs(1, int(cu[-1]), 2, 32, 128, "bf16", seed=152, s0="normal", num_seqs=len(lens))
    grads = gi.make_bwd_grads(1, int(cu[-1]), 2, 32, 128, "bf16", 152, with_dS=True, num_seqs=len(lens))
    print("case rect packed", flush=True)
    got = gpu_bwd(g, inp, grads, 64, cu=cu)
    ref = oracle.bwd(*(inp[n] for n in NAMES), grads["dout"], S0=inp["S0"], dS_final=grads["dS_final"],
                     cu_seqlens=cu)
    check(got, ref, TOL["bf16"], "rect packed")


@pytest.mark.parametrize("dtype,dk,dv,scalar", [("f32", 32, 64, False), ("bf16", 128, 64, True)])
def test_bwd_rect_heads_layer_prep(g, dtype, dk, dv, scalar):
    """dk != dv under layer prep: the widened key channels carry log-decay 0
    and zero q, k; the widened value channels zero v (their sigmoid gates
    then act on zeros)."""
    from oracle import layer_prep as lp
    raw = gi.make_layer_inputs(2, 100, 2, dk, dv, dtype, seed=960 + dk, s0="normal", scalar_beta=scalar)
    grads = gi.make_bwd_grads(2, 100, 2, dk, dv, dtype, seed=960 + dk)
    prep = lp.layer_prep(raw["q"], raw["k"], raw["alpha"], raw["b"], raw["w"])
    width = {"q": dk, "k": dk, "alpha": dk, "b": dk, "w": dv}
    full = {x: (prep[x][..., None] * np.ones(width[x]) if prep[x].ndim == 3 else prep[x]) for x in width}
    print(f"case rect layer prep {dtype} dk={dk} dv={dv} scalar={scalar}", flush=True)
    got = gpu_bwd_raw(g, raw, grads, 64, layer_prep=True)
    gp = oracle.bwd(full["q"], full["k"], raw["v"], full["alpha"], full["b"], full["w"], grads["dout"],
                    S0=raw["S0"], dS_final=grads["dS_final"])
    ref = lp.layer_prep_bwd(raw["q"], raw["k"], raw["alpha"], raw["b"], raw["w"], gp)
    ref["dS0"] = gp["dS0"]
    check(got, ref, TOL[dtype], f"rect layer prep {dtype} {dk}x{dv} scalar={scalar}")


PREPARED_CASES = [  # dtype, d, chunk, B, T, H, packed lengths (or None), gate layout
    ("bf16", 128, 64, 2, 300, 3, None, "channel"),       # plain two-pass, ragged last chunk
    ("f32", 64, 16, 1, 0, 2, [70, 0, 1, 130, 15], "channel"),   # packed, empty and 1-token sequences
    ("bf16", 64, 64, 1, 8192, 4, None, "channel"),      # one long sequence: the segment schedule
    ("bf16", 64, 64, 1, 0, 4, [9000, 8000], "channel"),       # packed long sequences: the segment schedule
    ("bf16", 32, 64, 2, 200, 2, None, "kda"),            # b = w = beta per (token, head)
]


@pytest.mark.parametrize("kept", [False, True], ids=["blocks", "blocks+states"])
@pytest.mark.parametrize("dtype,d,chunk,B,T,H,lens,gates", PREPARED_CASES)
def test_bwd_prepared_from_forward(g, dtype, d, chunk, B, T, H, lens, gates, kept):
    """A training step's forward (two-pass path) into the backward's own
    workspace, then the backward with the forward's blocks handed over (and,
    with ``kept``, the states the forward kept): the gradients and dS0 equal,
    bit for bit, those of the backward that recomputes them, and the
    forward's output is the plain forward's.  Where the backward takes the
    segment schedule (one or two long sequences) its own states come from
    the segment maps, so the kept states (one scan) agree with them up to
    rounding only: there the gradients are compared to 1e-2 of their
    largest magnitude (bfloat16 outputs, 2^-8 relative rounding, can flip
    by one unit)."""
    seed = 700 + d + H
    cu = None
    if lens is not None:
        cu = gi.cu_seqlens_from(lens)
        T = int(cu[-1])
    N = len(lens) if lens is not None else B
    inp = gi.make_chunk_inputs(B, T, H, d, d, dtype, seed, s0="normal",
                               **({"num_seqs": N} if lens is not None else {}))
    grads = gi.make_bwd_grads(B, T, H, d, d, dtype, seed, with_dS=True,
                              **({"num_seqs": N} if lens is not None else {}))
    print(f"prepared case {dtype} d={d} C={chunk} B={B} T={T} H={H} packed={lens is not None} gates={gates} "
          f"kept={kept}", flush=True)
    dev = {n: inp[n].cuda() for n in NAMES}
    if gates == "kda":
        beta = dev["b"][..., 0].contiguous()
        dev["b"] = beta
        dev["w"] = beta.clone()
    S0 = inp["S0"].cuda()
    dSf = grads["dS_final"].cuda()
    dout = grads["dout"].cuda()
    cud = None if cu is None else cu.cuda()
    ns = N if cu is not None else 0
    ws = torch.empty(g.bwd_workspace_bytes(B, T, H, d, d, ns, chunk, dev["q"].dtype), dtype=torch.uint8,
                     device="cuda")
    args = [dev[n] for n in NAMES]
    ref = g.chunk_bwd(*args, dout, S0=S0, dS_final=dSf, cu_seqlens=cud, chunk=chunk)
    ref = {k: v.clone() for k, v in ref.items() if v is not None}
    o_plain, Sf_plain = g.chunk_fwd(*args, S0=S0, cu_seqlens=cud, chunk=chunk, path="two_pass")
    ws.fill_(0xA5)  # the hand-over must not depend on what was there before the forward
    o, Sf = g.chunk_fwd(*args, S0=S0, cu_seqlens=cud, chunk=chunk, path="two_pass", workspace=ws,
                        keep_states=kept)
    got = g.chunk_bwd(*args, dout, S0=S0, dS_final=dSf, cu_seqlens=cud, chunk=chunk, workspace=ws, prepared=True,
                      states_kept=kept)
    torch.cuda.synchronize()
    assert torch.equal(o, o_plain) and torch.equal(Sf, Sf_plain)
    segment_shape = N * H <= 32 and (T if lens is None else T // N) >= 128 * chunk
    for name, x in ref.items():
        if kept and segment_shape:
            err = (got[name].float() - x.float()).abs().max().item()
            assert err <= 1e-2 * x.float().abs().max().item() + 1e-6, f"{name}: {err}"
        else:
            assert torch.equal(got[name], x), f"{name} differs from the recomputing backward"
