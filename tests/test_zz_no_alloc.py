"""GPU check of gdn2_chunk_fwd_noalloc, the allocation-free forward (its
intermediates live in the library's own device scratch), through the C ABI:
its outputs against gdn2_chunk_fwd's on the two-pass kernels for the same
inputs, on consecutive calls of different sizes (the scratch keeps the last
call's contents)."""
import ctypes

import numpy as np
import pytest
import torch

import gdn2_inputs as gi

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "alpha", "b", "w")
TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_07_amd as mod
    mod.lib()
    return mod


def rel_err(x, ref):
    x = x.double().cpu().numpy()
    ref = ref.double().cpu().numpy()
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


def run_pair(g, B, T, H, d, dtype, seed, chunk=64, cu=None, want_final=True):
    """Same inputs through both entry points; returns (o, S_final) of each."""
    n = None if cu is None else cu.numel() - 1
    inp = gi.make_chunk_inputs(B, T, H, d, d, dtype, seed=seed, s0="normal", num_seqs=n)
    dev = {x: inp[x].cuda() for x in NAMES}
    S0 = inp["S0"].cuda()
    cu_d = None if cu is None else cu.cuda()
    o_ref, S_ref = g.chunk_fwd(*(dev[x] for x in NAMES), S0=S0, cu_seqlens=cu_d, chunk=chunk, path="two_pass")
    N = B if cu is None else n
    o = torch.full_like(o_ref, float("nan"))
    Sf = torch.full((N, H, d, d), float("nan"), dtype=torch.float32, device="cuda") if want_final else None
    code = g.GDN2_BF16 if dtype == "bf16" else g.GDN2_F32
    st = g.lib().gdn2_chunk_fwd_noalloc(
        *(dev[x].data_ptr() for x in NAMES), S0.data_ptr(), None if cu_d is None else cu_d.data_ptr(),
        B, T, H, d, d, 0 if cu is None else n, chunk, code, 0, o.data_ptr(),
        None if Sf is None else Sf.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, g.lib().gdn2_last_error()
    torch.cuda.synchronize()
    return (o, Sf), (o_ref, S_ref)


def check(got, ref, dtype, label):
    (o, Sf), (o_ref, S_ref) = got, ref
    eo = rel_err(o.float(), o_ref.float())
    print(f"{label}: err_o={eo:.3e}", flush=True)
    assert eo <= TOL[dtype]
    assert torch.equal(o, o_ref), f"{label}: o differs from the two-pass entry point"
    if Sf is not None:
        es = rel_err(Sf, S_ref)
        print(f"{label}: err_S={es:.3e}", flush=True)
        assert es <= TOL[dtype]
        assert torch.equal(Sf, S_ref), f"{label}: S_final differs from the two-pass entry point"


def test_noalloc_matches_two_pass_on_consecutive_calls(g):
    # 1: larger than the scratch (2 x 4133 tokens x 16 heads, d = 128): runs
    #    in pieces of whole chunks, carried through S_final
    print("case noalloc 2x4133x16 d=128 bf16 (pieces)", flush=True)
    check(*run_pair(g, 2, 4096 + 37, 16, 128, "bf16", seed=61), "bf16", "pieces")
    # 2: a smaller call that fits the scratch in one go
    print("case noalloc 1x300x3 d=64 f32", flush=True)
    check(*run_pair(g, 1, 300, 3, 64, "f32", seed=62), "f32", "one call")
    # 3: larger than the scratch without S_final: the carry lives in the scratch
    print("case noalloc 1x9000x16 d=128 bf16, no S_final", flush=True)
    check(*run_pair(g, 1, 9000, 16, 128, "bf16", seed=63, want_final=False), "bf16", "pieces, no S_final")
    # 4: packed input with an empty sequence, then a smaller fixed-length call
    lens = [70, 0, 130, 33]
    print(f"case noalloc packed {lens} d=32 f32", flush=True)
    check(*run_pair(g, 1, sum(lens), 2, 32, "f32", seed=64, chunk=16, cu=gi.cu_seqlens_from(lens)), "f32",
          "packed")
    print("case noalloc 1x40x1 d=16 f32", flush=True)
    check(*run_pair(g, 1, 40, 1, 16, "f32", seed=65, chunk=16), "f32", "tiny")
