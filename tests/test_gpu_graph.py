"""HIP graphs of the library's entry points (MI355X only).

The library's calls launch kernels only (no allocation, copy, fill or
synchronisation), so a caller may capture them in a HIP graph and replay it.
Each test captures a sequence of calls, replays the graph several times with
the program's own eager work and synchronisations between the replays, and
checks every replay, bit for bit, against the same calls made eagerly: the
decode step's loop, the chunk forward, and a training step (forward, then
the backward on the forward's per-chunk blocks)."""
import pytest
import torch

import gdn2_inputs as gi

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "alpha", "b", "w")
GRADS = ("dq", "dk", "dv", "dalpha", "db", "dw", "dS0")
REPLAYS = 3


@pytest.fixture(scope="module")
def g():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_07_amd as mod
    mod.lib()
    return mod


def capture(fn):
    """fn() captured once in a HIP graph (after one eager warm-up on the
    capture's side stream, as torch asks)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        fn()
    torch.cuda.synchronize()
    return gr


def test_decode_steps_in_a_graph(g):
    """Four consecutive decode steps (distinct inputs, state updated in
    place) as one graph."""
    N, H, d, steps = 32, 4, 128, 4
    dd = gi.make_decode_inputs(N, H, d, d, "bf16", seed=77, steps=steps)
    x = {n: dd[n].cuda() for n in NAMES}
    S0 = dd["S"].cuda()
    print(f"graph decode N={N} H={H} d={d} steps={steps}", flush=True)

    S_e = S0.clone()
    o_e = [g.decode_step(*(x[n][t] for n in NAMES), S_e) for t in range(steps)]
    torch.cuda.synchronize()

    S_g = S0.clone()
    o_g = [torch.empty((N, H, d), dtype=torch.bfloat16, device="cuda") for _ in range(steps)]

    def run():
        for t in range(steps):
            g.decode_step(*(x[n][t] for n in NAMES), S_g, out=o_g[t])

    gr = capture(run)
    other = S0.clone()
    for r in range(REPLAYS):
        S_g.copy_(S0)
        gr.replay()
        # eager work of the program's own between replays
        g.decode_step(*(x[n][r % steps] for n in NAMES), other)
        torch.cuda.synchronize()
        assert torch.equal(S_g, S_e), f"replay {r}: state differs"
        for t in range(steps):
            assert torch.equal(o_g[t], o_e[t]), f"replay {r}: step {t} output differs"


@pytest.mark.parametrize("packed", [False, True])
def test_chunk_forward_in_a_graph(g, packed):
    H, d, C = 4, 64, 64
    if packed:
        cu = gi.cu_seqlens_from([300, 1, 0, 129])
        B, T, N = 1, int(cu[-1]), 4
        inp = gi.make_chunk_inputs(B, T, H, d, d, "bf16", seed=78, s0="normal", num_seqs=N)
        cud = cu.cuda()
    else:
        B, T, N, cud = 2, 450, 2, None
        inp = gi.make_chunk_inputs(B, T, H, d, d, "bf16", seed=79, s0="normal")
    x = [inp[n].cuda() for n in NAMES]
    S0 = inp["S0"].cuda()
    print(f"graph chunk_fwd packed={packed} B={B} T={T} H={H} d={d}", flush=True)
    ws = torch.empty(g.workspace_bytes(B, T, H, d, d, N if packed else 0, C, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    o_e, Sf_e = g.chunk_fwd(*x, S0=S0, cu_seqlens=cud, chunk=C)
    o_e, Sf_e = o_e.clone(), Sf_e.clone()
    o_g = torch.empty_like(o_e)
    Sf_g = torch.empty_like(Sf_e)
    gr = capture(lambda: g.chunk_fwd(*x, S0=S0, cu_seqlens=cud, chunk=C, out=o_g, S_final=Sf_g, workspace=ws))
    for r in range(REPLAYS):
        o_g.zero_()
        Sf_g.zero_()
        gr.replay()
        g.chunk_fwd(*x, S0=None, cu_seqlens=cud, chunk=C)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(Sf_g, Sf_e), f"replay {r} differs"


@pytest.mark.parametrize("kept", [False, True])
def test_training_step_in_a_graph(g, kept):
    """Forward (two-pass) into the backward's workspace, then the backward on
    the forward's blocks (and, with ``kept``, its kept states): one graph."""
    B, T, H, d, C = 2, 300, 3, 128, 64
    inp = gi.make_chunk_inputs(B, T, H, d, d, "bf16", seed=80, s0="normal")
    grads = gi.make_bwd_grads(B, T, H, d, d, "bf16", seed=80, with_dS=True)
    x = [inp[n].cuda() for n in NAMES]
    S0, dout, dSf = inp["S0"].cuda(), grads["dout"].cuda(), grads["dS_final"].cuda()
    print(f"graph training step B={B} T={T} H={H} d={d} kept={kept}", flush=True)
    ws = torch.empty(g.bwd_workspace_bytes(B, T, H, d, d, 0, C, torch.bfloat16), dtype=torch.uint8, device="cuda")

    o_e, Sf_e = g.chunk_fwd(*x, S0=S0, chunk=C)
    o_e, Sf_e = o_e.clone(), Sf_e.clone()
    ref = g.chunk_bwd(*x, dout, S0=S0, dS_final=dSf, chunk=C)
    ref = {k: v.clone() for k, v in ref.items()}

    o_g, Sf_g = torch.empty_like(o_e), torch.empty_like(Sf_e)
    gout = {k: torch.empty_like(v) for k, v in ref.items()}

    def step():
        g.chunk_fwd(*x, S0=S0, chunk=C, out=o_g, S_final=Sf_g, workspace=ws, path="two_pass", keep_states=kept)
        g.chunk_bwd(*x, dout, S0=S0, dS_final=dSf, chunk=C, workspace=ws, out=gout, prepared=True,
                    states_kept=kept)

    gr = capture(step)
    for r in range(REPLAYS):
        for v in gout.values():
            v.zero_()
        ws.fill_(0)
        gr.replay()
        g.chunk_bwd(*x, dout, chunk=C)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(Sf_g, Sf_e), f"replay {r}: forward differs"
        for name in GRADS:
            assert torch.equal(gout[name], ref[name]), f"replay {r}: {name} differs"
