"""Heads whose key and value widths differ (dk != dv) against the float64
oracle: the chunked paths (run on d = max(dk, dv) with the narrower side
widened in the workspace), the token-by-token path and the decode step
(both built for every (dk, dv) pair)."""
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
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-30))


def check(o, Sf, o_ref, S_ref, tol, label):
    eo, es = rel_err(o, o_ref), rel_err(Sf, S_ref)
    print(f"{label} err_o={eo:.3e} err_S={es:.3e}", flush=True)
    assert o.shape == o_ref.shape and Sf.shape == S_ref.shape, label
    assert eo <= tol, f"{label}: o error {eo:.3e} > {tol}"
    assert es <= tol, f"{label}: S_final error {es:.3e} > {tol}"


CASES = [("f32", 16, 64, 16, 2, 100, 3, "auto"), ("bf16", 128, 64, 64, 2, 200, 4, "auto"),
         ("bf16", 64, 128, 64, 2, 150, 3, "auto"), ("bf16", 16, 128, 64, 1, 300, 2, "two_pass"),
         ("f32", 128, 32, 16, 2, 70, 2, "two_pass"), ("bf16", 32, 64, 64, 3, 130, 2, "fused"),
         ("f32", 64, 16, 16, 2, 90, 3, "fused"), ("bf16", 128, 16, 64, 2, 129, 2, "recurrent"),
         ("f32", 16, 32, 16, 2, 33, 2, "recurrent")]


@pytest.mark.parametrize("dtype,dk,dv,chunk,B,T,H,path", CASES)
def test_rect_heads_forward(g, dtype, dk, dv, chunk, B, T, H, path):
    inp = gi.make_chunk_inputs(B, T, H, dk, dv, dtype, seed=300 + dk + 3 * dv + T, s0="normal")
    print(f"case rect {dtype} dk={dk} dv={dv} C={chunk} B={B} T={T} H={H} {path}", flush=True)
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    d = {n: inp[n].cuda() for n in NAMES}
    o, Sf = g.chunk_fwd(*(d[n] for n in NAMES), S0=inp["S0"].cuda(), chunk=chunk,
                        path="auto" if path == "recurrent" else path, recurrent=path == "recurrent")
    torch.cuda.synchronize()
    check(o.float().cpu().numpy(), Sf.cpu().numpy(), o_ref, S_ref, TOL[dtype], f"rect {dtype} {dk}x{dv} {path}")


def test_rect_heads_packed_rule_r1_gates(g):
    """Packed sequences (empty and one-token ones included), rule R1, and
    per-(token, head) gates with layer prep, each with dk != dv."""
    lens = [70, 0, 1, 64, 130, 15]
    cu = gi.cu_seqlens_from(lens)
    inp = gi.make_chunk_inputs(1, int(cu[-1]), 3, 64, 128, "bf16", seed=311, s0="normal", num_seqs=len(lens))
    d = {n: inp[n].cuda() for n in NAMES}
    for rule in ("R5", "R1"):
        o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"], cu_seqlens=cu, rule=rule)
        print(f"case rect packed {rule}", flush=True)
        o, Sf = g.chunk_fwd(*(d[n] for n in NAMES), S0=inp["S0"].cuda(), cu_seqlens=cu.cuda(), chunk=64, rule=rule)
        torch.cuda.synchronize()
        check(o.float().cpu().numpy(), Sf.cpu().numpy(), o_ref, S_ref, TOL["bf16"], f"rect packed {rule}")
    # b and w per (token, head): the KDA reduction with dk != dv
    inp = gi.make_chunk_inputs(2, 150, 2, 128, 64, "f32", seed=312, s0="normal", scalar_beta=True)
    o_ref, S_ref = oracle.fwd(*(inp[n] for n in NAMES), S0=inp["S0"])
    compact = dict(inp, b=inp["b"][..., 0].contiguous(), w=inp["w"][..., 0].contiguous())
    print("case rect KDA gates", flush=True)
    o, Sf = g.chunk_fwd(*(compact[n].cuda() for n in NAMES), S0=inp["S0"].cuda(), chunk=64)
    torch.cuda.synchronize()
    check(o.float().cpu().numpy(), Sf.cpu().numpy(), o_ref, S_ref, TOL["f32"], "rect KDA gates")
    # layer prep: raw q, k, b and w logits, float32 natural-log decay
    from oracle import layer_prep as lp
    raw = gi.make_layer_inputs(2, 140, 3, 32, 128, "bf16", seed=313, s0="normal")
    prep = lp.layer_prep(raw["q"], raw["k"], raw["alpha"], raw["b"], raw["w"])
    o_ref, S_ref = oracle.fwd(prep["q"], prep["k"], raw["v"], prep["alpha"], prep["b"], prep["w"], S0=raw["S0"])
    print("case rect layer prep", flush=True)
    o, Sf = g.chunk_fwd(*(raw[n].cuda() for n in NAMES), S0=raw["S0"].cuda(), chunk=64, layer_prep=True)
    torch.cuda.synchronize()
    check(o.float().cpu().numpy(), Sf.cpu().numpy(), o_ref, S_ref, TOL["bf16"], "rect layer prep")


@pytest.mark.parametrize("dtype,dk,dv", [("f32", 64, 128), ("bf16", 128, 16), ("f32", 16, 32)])
def test_rect_heads_decode(g, dtype, dk, dv):
    dd = gi.make_decode_inputs(5, 3, dk, dv, dtype, seed=320 + dk + dv, steps=6)
    S_gpu = dd["S"].cuda()
    S_ref = dd["S"].double().numpy()
    for t in range(6):
        step = {n: dd[n][t].contiguous() for n in NAMES}
        o = g.decode_step(*(step[n].cuda() for n in NAMES), S_gpu)
        o_ref, S_ref = oracle.decode(*(step[n] for n in NAMES), S_ref)
        torch.cuda.synchronize()
        check(o.float().cpu().numpy(), S_gpu.cpu().numpy(), o_ref, S_ref, TOL[dtype], f"rect decode {dk}x{dv} t={t}")
