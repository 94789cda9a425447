"""Benchmark of the GDN-2 forward hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one gdn2_chunk_fwd call over the 1.3B-scale training-shape layer
(B=8, T=4096, H=16, dk=dv=128, chunk 64, bf16 inputs, fp32 state and
accumulation, S0 = 0) with the inputs already resident in HBM.  `value` is
tokens/s over the K timed steps (bracketed by device synchronisations).

In the same run (reported next to the headline, not in `value`):
  * per-kernel durations from HIP events recorded on the launch stream
    (libgdn2's timing hooks) and the roofline of the dominant kernel;
  * the path as a whole against its algorithmic bytes and FLOPs;
  * the T sweep at B*T = 32768 (T = 2K .. 32K) and the packed-sequence
    workload (lengths uniform in [256, 8192], 32768 tokens);
  * the decode step (256 sequences x 16 heads, 256 MiB fp32 state updated in
    place): eager launches and HIP graph replays of the same loop, and its
    kernel warm and with two alternating state buffers (512 MiB, more than
    the 256 MB last-level cache);
  * the same layer as KDA (b = w = beta per token and head) and as Gated
    DeltaNet (also a per-(token, head) decay), and GDN-2's time over KDA's;
  * the same layer under the alternative reading R1 (chunked two-pass path);
  * the chunked backward (gdn2_chunk_bwd) on the same layer: its time per
    step, per-kernel durations and the roofline of its dominant kernel, and
    a training step (the forward, then the backward on the forward's
    per-chunk blocks);
  * a context-parallel split of one 32768-token sequence into 8 segments:
    the per-rank segment map and re-run against the serial forward, and all
    eight on this GPU with the scan of the maps;
  * the CPU oracle timed on a bounded sample of the same workload.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gdn2_inputs as gi  # noqa: E402

NAMES = ("q", "k", "v", "alpha", "b", "w")
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 matrix peak, TFLOP/s


def flops_per_token_head(d: int, C: int) -> float:
    """Algorithmic FLOPs of the chunked form per token and head (dk = dv = d):
    A and P products, the triangular inverse, W/Ut, the state read-outs and the
    state update, counted once (no dense-tile padding)."""
    return 2.0 * (3 * d * d + ((3 * C - 1) / 2) * d + C * d + C * C / 6)


# Algorithmic HBM bytes per token and head (bf16 elements, d = 128):
#   path : read q, k, v, alpha, b, w once, write o once
#   prep : read the six inputs, write -W, Q', Kbar^T, Ut (bf16), the lower
#          triangle of P (C/16 (C/16 + 1) / 2 tiles of 16 x 16 per chunk) and
#          gamma_C (fp32, one d-vector per chunk)
#   scan : read -W, Q', Kbar^T, Ut, P and gamma_C, write o
#   fused: the path itself (inputs once, o once)
def p_bytes_per_token_head(C: int, elem: int = 2) -> float:
    nb = C // 16
    return nb * (nb + 1) / 2 * 256 * elem / C


def bytes_per_token_head(d: int, C: int, elem: int = 2) -> dict:
    gam = d * 4 / C
    pb = p_bytes_per_token_head(C, elem)
    return {
        "path": 6 * d * elem + d * elem,
        "chunk_fused": 6 * d * elem + d * elem,
        "chunk_prep": 6 * d * elem + 4 * d * elem + pb + gam,
        "chunk_scan": 4 * d * elem + pb + gam + d * elem,
    }


# Algorithmic HBM bytes per token and head of the backward's kernels (bf16
# elements; a state crosses HBM as one fragment-tile copy of d*d elements
# per chunk):
#   path         : read q, k, v, alpha, b, w and dL/do once, write six gradients
#   chunk_states : read -W, Kbar^T, Ut and gamma_C, write the entering state
#   bwd_dstate   : read -W, Q', Kbar^T, gamma_C and dL/do, write the leaving-state gradient
#   bwd_grad     : read the six inputs, dL/do, the state and its gradient, write six gradients
def bwd_bytes_per_token_head(d: int, C: int, elem: int = 2) -> dict:
    gam = d * 4 / C
    st = d * d * elem / C
    pb = p_bytes_per_token_head(C, elem)
    return {
        "path": 7 * d * elem + 6 * d * elem,
        "chunk_prep": 6 * d * elem + 4 * d * elem + pb + gam,
        "chunk_states": 3 * d * elem + gam + st,
        "bwd_dstate": 4 * d * elem + gam + st,
        "bwd_grad": 7 * d * elem + 2 * st + 6 * d * elem,
    }


# The sources that define the chunked forward's kernels (prep and scan):
# their file, the per-chunk phases, the device helpers and the argument
# block.  A counter record stays valid while these are unchanged.
KERNEL_SOURCES = ("gdn2_chunk.hip", "gdn2_wy.hpp", "gdn2_device.hpp", "gdn2_kernels.hpp")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gated_delta_rule_07_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def event_us(fn, steps: int, warmup: int) -> float:
    """Average time of one call of fn in microseconds, from two HIP events
    recorded on torch's current stream (the stream the library launches on)
    around `steps` calls."""
    for _ in range(warmup):
        fn()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start.record()
    for _ in range(steps):
        fn()
    t_end.record()
    t_end.synchronize()
    return t_start.elapsed_time(t_end) * 1e3 / steps


def timed_steps(fn, steps: int, warmup: int) -> float:
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def cpu_baseline(inp: dict, H: int, budget_s: float) -> dict:
    """The oracle on all (batch, head) units of the workload but only the first
    T' tokens of each sequence, T' chosen so the run takes roughly budget_s."""
    import oracle
    threads = oracle.max_threads()
    B = inp["q"].shape[0]

    def run(Tp):
        sub = {x: inp[x][:, :Tp].contiguous() for x in NAMES}
        t0 = time.perf_counter()
        oracle.fwd(*(sub[x] for x in NAMES))
        return time.perf_counter() - t0

    Tc = 64
    dt = run(Tc)
    rate = B * H * Tc / dt                     # token-heads per second
    T = inp["q"].shape[1]
    Tp = int(max(64, min(T, (rate * budget_s / (B * H)) // 64 * 64)))
    reps, total = 0, 0.0
    while total < budget_s and reps < 64:      # repeat the sample until the budget is spent
        total += run(Tp)
        reps += 1
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": B * Tp * reps / total, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu,
            "sample": f"float64 token-by-token oracle on all {B}x{H} (batch, head) units of the "
                      f"workload, first {Tp} of {T} tokens each, {reps} run(s), {total:.1f} s"}


def load_traffic() -> dict | None:
    """HBM bytes per launch of the forward's kernels measured with rocprofv3
    counters (FETCH_SIZE and WRITE_SIZE, scaled by a device copy of known
    size), if they were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_chunk_fwd_layer_8x4096x16_d128.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec


def host_info() -> dict:
    """CPU model and core count of the host, GPU name and architecture."""
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    p = torch.cuda.get_device_properties(0)
    arch = getattr(p, "gcnArchName", "")
    # the device name comes from libdrm's marketing-name table, which some
    # hosts lack: then say so rather than print nothing
    name = p.name or f"{arch.split(':')[0]} (no marketing-name table on this host)"
    return {"cpu_model": cpu, "host_cpus": os.cpu_count(), "gpu_name": name,
            "gpu_arch": arch, "compute_units": p.multi_processor_count,
            "gpu_memory_gib": round(p.total_memory / 2**30, 1), "gpu_clocks": gpu_clocks()}


def gpu_clocks():
    """The current clock levels rocm-smi reports for the first GPU (read
    once, right after the headline's timed steps, while the clocks are
    still up), or None when it cannot tell."""
    import json
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=10)
        cards = json.loads(r.stdout)
        card = cards[sorted(cards)[0]]
        return {k.strip(" :"): v for k, v in card.items() if "clock" in k.lower() or "clk" in k.lower()}
    except Exception:  # absent tool, other output format: the line carries None
        return None


def rel_err(x: np.ndarray, ref: np.ndarray) -> float:
    """max |x - ref| / max |ref| over the whole tensor."""
    return float(np.max(np.abs(x - ref)) / max(float(np.max(np.abs(ref))), 1e-30))


# Algorithmic HBM bytes of the segment-map kernel per token and head: read
# -W, Kbar^T and Ut (bf16) and gamma_C (fp32 per chunk); the two maps it
# writes (2 d^2 fp32 per segment and head) are added per launch.  FLOPs: the
# products Z = Ut - W S and S <- gamma S + Kbar^T Z, 4 d^2 per token for each
# of Phi and Psi.
def segmap_bytes_per_token_head(d: int, C: int, elem: int = 2) -> float:
    return 3 * d * elem + d * 4 / C


def context_parallel(g, dev: dict, H: int, d: int, C: int, path: str) -> dict:
    """The 32768-token stream of the packed workload as ONE sequence cut
    into 8 segments of 4096 tokens (an 8-way context-parallel split).  Per
    rank: the segment's map (prep + segment-map kernel) and its re-run from
    the true entering state (gdn2_chunk_fwd, in full, and on the workspace
    the map left: the scan alone), against the serial forward of the same
    4096 x 16 share.  On one GPU: all 8 maps in one call, the scan
    of the maps, the 8 re-runs in one packed call, against the forward of the
    whole 32768-token sequence."""
    G, L = 8, 4096
    res = {"workload": "one 32768-token sequence, H=16, d=128, bf16, cut into 8 segments of 4096",
           "per_rank_shape": {"T": L, "H": H}}
    rank = {x: dev[x][0:1] for x in NAMES}                    # [1, 4096, H, d]
    ws1 = torch.empty(g.workspace_bytes(1, L, H, d, d, 0, C, torch.bfloat16), dtype=torch.uint8, device="cuda")
    Phi1 = torch.empty((1, H, d, d), dtype=torch.float32, device="cuda")
    Psi1 = torch.empty_like(Phi1)
    o1 = torch.empty((1, L, H, d), dtype=torch.bfloat16, device="cuda")
    Sf1 = torch.empty((1, H, d, d), dtype=torch.float32, device="cuda")
    S_in1 = torch.zeros((1, H, d, d), dtype=torch.float32, device="cuda")

    def rank_map():
        g.segment_map(*(rank[x] for x in NAMES), chunk=C, workspace=ws1, out=(Phi1, Psi1))

    def rank_fwd(S0):
        g.chunk_fwd(*(rank[x] for x in NAMES), S0=S0, chunk=C, out=o1, S_final=Sf1, workspace=ws1, path=path)

    g.profile_enable(True)
    g.profile_read(reset=True)
    sec_map = timed_steps(rank_map, 20, 3)
    prof = g.profile_read(reset=True)
    g.profile_enable(False)
    kern = {k: {"avg_us": 1e3 * ms / n, "launches": n} for k, (ms, n) in prof.items()}
    sec_rerun = timed_steps(lambda: rank_fwd(S_in1), 20, 3)
    # the re-run on the workspace the map left (GDN2_FLAG_PREPARED): scan only
    rank_map()
    sec_rerun_p = timed_steps(lambda: g.chunk_fwd(*(rank[x] for x in NAMES), S0=S_in1, chunk=C, out=o1,
                                                  S_final=Sf1, workspace=ws1, prepared=True), 20, 3)
    sec_serial = timed_steps(lambda: rank_fwd(None), 20, 3)
    sm_us = kern["segment_map"]["avg_us"]
    tok_heads = L * H
    sm_bytes = segmap_bytes_per_token_head(d, C) * tok_heads + 2 * H * d * d * 4
    sm_flops = 8.0 * d * d * tok_heads
    res["per_rank"] = {
        "map_ms": round(sec_map * 1e3, 4), "rerun_ms": round(sec_rerun * 1e3, 4),
        "serial_forward_ms": round(sec_serial * 1e3, 4),
        "map_plus_rerun_over_serial": round((sec_map + sec_rerun) / sec_serial, 3),
        "prepared_rerun_ms": round(sec_rerun_p * 1e3, 4),
        "map_plus_prepared_rerun_over_serial": round((sec_map + sec_rerun_p) / sec_serial, 3),
        "kernels": kern,
        "segment_map_roofline": {"bound": "hbm", "achieved": round(sm_bytes / (sm_us * 1e-6) / 1e9, 1),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(sm_bytes / (sm_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                 "algorithmic_bytes_per_launch": int(sm_bytes),
                                 "tflops": round(sm_flops / (sm_us * 1e-6) / 1e12, 2)},
    }
    del ws1

    # all eight segments on this one GPU
    cu = gi.cu_seqlens_from([L] * G).cuda()
    full = {x: dev[x].view(1, G * L, H, d) for x in NAMES}
    wsG = torch.empty(g.workspace_bytes(1, G * L, H, d, d, G, C, torch.bfloat16), dtype=torch.uint8, device="cuda")
    PhiG = torch.empty((G, H, d, d), dtype=torch.float32, device="cuda")
    PsiG = torch.empty_like(PhiG)
    S_inG = torch.empty_like(PhiG)
    oG = torch.empty((1, G * L, H, d), dtype=torch.bfloat16, device="cuda")
    SfG = torch.empty_like(PhiG)
    ws_seq = torch.empty(g.workspace_bytes(1, G * L, H, d, d, 0, C, torch.bfloat16), dtype=torch.uint8,
                         device="cuda")
    Sf_seq = torch.empty((1, H, d, d), dtype=torch.float32, device="cuda")

    def all_maps():
        g.segment_map(*(full[x] for x in NAMES), cu_seqlens=cu, chunk=C, workspace=wsG, out=(PhiG, PsiG))

    def combine():
        g.segment_combine(PhiG, PsiG, None, want_final=False, out=S_inG)

    def reruns():
        g.chunk_fwd(*(full[x] for x in NAMES), S0=S_inG, cu_seqlens=cu, chunk=C, out=oG, S_final=SfG,
                    workspace=wsG, path=path)

    def whole():
        g.chunk_fwd(*(full[x] for x in NAMES), chunk=C, out=oG, S_final=Sf_seq, workspace=ws_seq, path=path)

    def whole_serial():
        g.chunk_fwd(*(full[x] for x in NAMES), chunk=C, out=oG, S_final=Sf_seq, workspace=ws_seq, path="two_pass")

    g.profile_enable(True)
    g.profile_read(reset=True)
    sec_comb = timed_steps(combine, 20, 3)
    cprof = g.profile_read(reset=True)
    g.profile_enable(False)
    def reruns_prepared():
        g.chunk_fwd(*(full[x] for x in NAMES), S0=S_inG, cu_seqlens=cu, chunk=C, out=oG, S_final=SfG,
                    workspace=wsG, prepared=True)

    sec_all = timed_steps(lambda: (all_maps(), combine(), reruns()), 10, 2)
    sec_all_p = timed_steps(lambda: (all_maps(), combine(), reruns_prepared()), 10, 2)
    sec_whole = timed_steps(whole, 10, 2)
    sec_serial_w = timed_steps(whole_serial, 10, 2)
    # the backward of the same sequence (its scans take the segment schedule too)
    grads = gi.make_bwd_grads(1, G * L, H, d, d, "bf16", seed=5, with_dS=False)
    dout = grads["dout"].cuda()
    wsb = torch.empty(g.bwd_workspace_bytes(1, G * L, H, d, d, 0, C, torch.bfloat16), dtype=torch.uint8,
                      device="cuda")
    gout = {n: torch.empty_like(full[x]) for n, x in zip(("dq", "dk", "dv", "dalpha", "db", "dw"), NAMES)}
    gout["dS0"] = torch.empty((1, H, d, d), dtype=torch.float32, device="cuda")
    sec_bwd = timed_steps(lambda: g.chunk_bwd(*(full[x] for x in NAMES), dout, chunk=C, workspace=wsb, out=gout), 5, 2)
    del wsb, gout, dout
    res["one_gpu"] = {
        "maps_combine_reruns_ms": round(sec_all * 1e3, 4),
        "maps_combine_prepared_reruns_ms": round(sec_all_p * 1e3, 4),
        "whole_sequence_serial_scan_ms": round(sec_serial_w * 1e3, 4),
        "whole_sequence_default_path_ms": round(sec_whole * 1e3, 4),
        "whole_sequence_backward_ms": round(sec_bwd * 1e3, 4),
        "prepared_over_serial": round(sec_all_p / sec_serial_w, 3),
        "combine_kernel_us": round(1e3 * cprof["segment_combine"][0] / cprof["segment_combine"][1], 2),
        "exchange_bytes_per_rank": 2 * H * d * d * 4,
    }
    return res


def configs_table(g) -> dict:
    """Every workload once (part of the oracle leg, ``--configs``): GPU time
    (HIP-synchronised wall time per call after warm-up), parity against the
    oracle (max |gpu - oracle| / max |oracle| of o and S_final, every
    element) and the oracle's own time on the host's cores."""
    import oracle
    out = {}

    def timed(fn, budget_s=0.3):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            fn()
            n += 1
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / n

    fwd_cases = [("tiny_1x64x1_d16", None), ("small_2x512x4_d64", None), ("small_2x512x4_d64", "kda"),
                 ("layer_8x4096x16_d128", None), ("packed_32768x16_d128", None)]
    for name, variant in fwd_cases:
        c = gi.WORKLOADS[name]
        cu = None
        if c.get("packed"):
            lens = gi.packed_lengths(c["seed"])
            cu = gi.cu_seqlens_from(lens)
            inp = gi.make_chunk_inputs(1, c["T"], c["H"], c["dk"], c["dv"], c["dtype"], c["seed"], s0=c["s0"],
                                       num_seqs=len(lens))
        else:
            inp = gi.make_chunk_inputs(c["B"], c["T"], c["H"], c["dk"], c["dv"], c["dtype"], c["seed"], s0=c["s0"],
                                       scalar_beta=(variant == "kda"))
        dev = {x: inp[x].cuda() for x in NAMES}
        if variant == "kda":  # b = w = beta per (token, head): the KDA input layout
            dev = dict(dev, b=dev["b"][..., 0].contiguous(), w=dev["w"][..., 0].contiguous())
        S0 = inp["S0"].cuda() if inp.get("S0") is not None else None
        cud = cu.cuda() if cu is not None else None
        fn = lambda: g.chunk_fwd(*(dev[x] for x in NAMES), S0=S0, cu_seqlens=cud, chunk=c["chunk"])
        sec = timed(fn)
        o, Sf = fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        o_ref, S_ref = oracle.fwd(*(inp[x] for x in NAMES), S0=inp.get("S0"), cu_seqlens=cu)
        t_or = time.perf_counter() - t0
        tok = int(o.shape[0] * o.shape[1])
        key = name + ("_kda_gates" if variant else "")
        out[key] = {"dtype": c["dtype"], "gpu_ms": round(sec * 1e3, 4), "tokens_per_s": round(tok / sec, 1),
                    "tflops": round(flops_per_token_head(c["dk"], c["chunk"]) * tok * c["H"] / sec / 1e12, 3),
                    "err_o": rel_err(o.float().cpu().numpy(), o_ref), "err_S": rel_err(Sf.cpu().numpy(), S_ref),
                    "oracle_s": round(t_or, 3)}
        del dev, o, Sf
    c = gi.WORKLOADS["decode_256x16_d128"]
    dd = gi.make_decode_inputs(c["N"], c["H"], c["dk"], c["dv"], "bf16", c["seed"], steps=c["steps"])
    S_gpu = dd["S"].cuda()
    ddev = {x: dd[x].cuda() for x in NAMES}
    outs = [g.decode_step(*(ddev[x][t] for x in NAMES), S_gpu) for t in range(c["steps"])]
    torch.cuda.synchronize()
    S_ref = dd["S"].double().numpy()
    eo, t0 = 0.0, time.perf_counter()
    for t in range(c["steps"]):
        o_ref, S_ref = oracle.decode(*(dd[x][t] for x in NAMES), S_ref)
        eo = max(eo, rel_err(outs[t].float().cpu().numpy(), o_ref))
    t_or = (time.perf_counter() - t0) / c["steps"]
    out["decode_256x16_d128"] = {"dtype": "bf16", "steps": c["steps"], "err_o_max_over_steps": eo,
                                 "err_S_after_steps": rel_err(S_gpu.cpu().numpy(), S_ref),
                                 "oracle_ms_per_step": round(t_or * 1e3, 2)}
    out["oracle_cores"] = oracle.max_threads()
    return out


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # about 0.1 s of warm-up: the first milliseconds of load run at lower
    # clocks (the prep kernel measured 354 us cold against 310 us warm)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-extras", action="store_true", help="headline workload only")
    ap.add_argument("--path", default="auto", choices=["auto", "fused", "two_pass"],
                    help="chunked kernels to time (default: the library's own choice)")
    ap.add_argument("--configs", action="store_true",
                    help="also run every workload once against the oracle (GPU time, error, oracle time)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(every (sequence, head) is independent, and a long sequence splits through its segment maps)",
              file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    import gated_delta_rule_07_amd as g

    B, T, H, d, C = 8, 4096, 16, 128, 64
    inp = gi.make_chunk_inputs(B, T, H, d, d, "bf16", seed=2, s0=None)
    dev = {x: inp[x].cuda() for x in NAMES}
    o = torch.empty((B, T, H, d), dtype=torch.bfloat16, device="cuda")
    Sf = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")
    # one workspace for the headline and every T of the sweep (a single long
    # sequence also takes the segment schedule's maps)
    ws = torch.empty(max([g.workspace_bytes(B, T, H, d, d, 0, C, torch.bfloat16)] +
                         [g.workspace_bytes(32768 // Ts, Ts, H, d, d, 0, C, torch.bfloat16) for Ts in gi.SWEEP_T]),
                     dtype=torch.uint8, device="cuda")

    def step():
        g.chunk_fwd(*(dev[x] for x in NAMES), chunk=C, out=o, S_final=Sf, workspace=ws,
                    path=args.path)

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # per-kernel durations first, in passes of their own (so that the
    # headline below is timed on the clocks a running workload holds: the
    # first milliseconds of load after idle run about 9 % slower): the library's HIP events
    # around every launch (an event between the two kernels delays the next
    # launch, the prep's by about 15 %)
    g.profile_enable(True)
    g.profile_read(reset=True)
    sec_hooks = timed_steps(step, args.steps, 3)
    prof = g.profile_read(reset=True)
    g.profile_enable(False)
    kern_hooked = {k: {"avg_us": 1e3 * ms / n, "launches": n} for k, (ms, n) in prof.items()}
    kern = kern_hooked
    duration_method = "library HIP events around every launch"
    if set(kern_hooked) == {"chunk_prep", "chunk_scan"}:
        # without per-launch events: HIP events around K whole steps and
        # around K runs of the scan alone on the workspace the last step
        # filled (prepared mode, same blocks); the prep is the difference
        def scan_only():
            g.chunk_fwd(*(dev[x] for x in NAMES), chunk=C, out=o, S_final=Sf, workspace=ws,
                        path=args.path, prepared=True)
        full_us = event_us(step, args.steps, 20)
        scan_us = event_us(scan_only, args.steps, 20)
        kern = {"chunk_prep": {"avg_us": full_us - scan_us, "launches": args.steps},
                "chunk_scan": {"avg_us": scan_us, "launches": args.steps}}
        duration_method = ("HIP events on the launch stream around K steps and around K scan-only "
                           "runs on the filled workspace; prep = step - scan")

    # the headline: W warm-up steps, then K timed steps, the library's timing hooks off
    sec = timed_steps(step, args.steps, args.warmup)
    # the timed output against the oracle (every element of o and S_final)
    o_gpu = o.float().cpu().numpy()
    S_gpu = Sf.cpu().numpy()

    tok_heads = B * T * H
    fl = flops_per_token_head(d, C) * tok_heads
    byt = bytes_per_token_head(d, C)
    path_bytes = byt["path"] * tok_heads
    dominant = max(kern, key=lambda k: kern[k]["avg_us"])
    dom_us = kern[dominant]["avg_us"]
    achieved = path_bytes / (dom_us * 1e-6) / 1e9
    own_bytes = byt[dominant] * tok_heads
    own_achieved = own_bytes / (dom_us * 1e-6) / 1e9
    tr = load_traffic()
    traffic = tr["kernels"][dominant]["bytes_per_launch"] if tr and dominant in tr["kernels"] else None
    step_traffic = (sum(tr["kernels"][k]["bytes_per_launch"] for k in kern if k in tr["kernels"])
                    if tr and all(k in tr["kernels"] for k in kern) else None)
    # roofline of the dominant kernel: the path's algorithmic bytes (1792 B
    # per token-head: six bf16 inputs read once, o written once) over that
    # kernel's average launch time; the kernel's own bytes (its inputs and
    # outputs, workspace included) are reported beside it
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": dominant, "duration_us": round(dom_us, 2), "duration_method": duration_method,
                "algorithmic_bytes_per_launch": int(path_bytes),
                "algorithmic_bytes_per_token_head": byt["path"], "token_heads_per_launch": tok_heads,
                "kernel_own": {"bytes_per_launch": int(own_bytes), "achieved": round(own_achieved, 1),
                               "frac": round(own_achieved / HBM_PEAK_GBS, 4)},
                "traffic_over_algorithmic": (round(step_traffic / path_bytes, 3) if step_traffic else None)}

    out = {
        "metric": "GDN-2 chunk fwd tokens/s + % bf16 MFMA peak (H16 d128 T4K); decode % HBM",
        "value": round(B * T / sec, 1),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(sec * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "GDN-2 chunked forward, 1.3B-scale layer shape", "B": B, "T": T,
                   "H": H, "dk": d, "dv": d, "chunk": C, "inputs": "bf16", "state": "fp32",
                   "S0": "zero", "parallelism": "single GPU"},
        "roofline": roofline,
        "path": {"tflops": round(fl / sec / 1e12, 2),
                 "mfma_frac": round(fl / sec / 1e12 / BF16_PEAK_TFLOPS, 4),
                 "algorithmic_bytes": int(path_bytes),
                 "hbm_frac": round(path_bytes / sec / 1e9 / HBM_PEAK_GBS, 4),
                 "flops_per_token_head": flops_per_token_head(d, C),
                 "step_traffic_bytes": step_traffic},
        "kernels": kern,
        "kernels_event_hooks": kern_hooked,
        "ms_per_step_with_timing_hooks": round(sec_hooks * 1e3, 4),
        "host": host_info(),
    }
    if not args.no_cpu:
        import oracle
        t0 = time.perf_counter()
        o_ref, S_ref = oracle.fwd(*(inp[x] for x in NAMES))
        eo, es = rel_err(o_gpu, o_ref), rel_err(S_gpu, S_ref)
        out["max_err_o"] = eo
        out["max_err_S"] = es
        out["parity"] = {"max_err_o": eo, "max_err_S": es, "tol": 2e-2,
                         "metric": "max |gpu - oracle| / max |oracle| over every element of the timed step's "
                                   "o and S_final",
                         "oracle": "float64 token-by-token recurrence, all 128 (batch, head) units",
                         "oracle_s": round(time.perf_counter() - t0, 2)}
        del o_ref, S_ref
    del o_gpu, S_gpu

    if not args.no_extras:
        # T sweep at B*T = 32768 and the packed workload reuse the same tokens
        # (the oracle above leaves the GPU idle for seconds: every point first
        # runs untimed for about 0.15 s, and the points are timed in 3
        # interleaved rounds of 20 steps, the median reported)
        sweep_fns = {}
        for Ts in gi.SWEEP_T:
            Bs = 32768 // Ts
            view = {x: dev[x].view(Bs, Ts, H, d) for x in NAMES}
            Sf2 = torch.empty((Bs, H, d, d), dtype=torch.float32, device="cuda")
            sweep_fns[Ts] = (lambda view=view, o2=o.view(Bs, Ts, H, d), Sf2=Sf2:
                             g.chunk_fwd(*(view[x] for x in NAMES), chunk=C, out=o2, S_final=Sf2, workspace=ws,
                                         path=args.path))
        sweep_secs = {Ts: [] for Ts in gi.SWEEP_T}
        for _ in range(3):
            for Ts, fn in sweep_fns.items():
                sweep_secs[Ts].append(timed_steps(fn, 20, 300))
        sweep = {str(Ts): round(32768 / float(np.median(v)), 1) for Ts, v in sweep_secs.items()}
        del sweep_fns
        vals = list(sweep.values())
        out["sweep_tokens_per_s"] = sweep
        out["sweep_flatness_min_over_max"] = round(min(vals) / max(vals), 3)

        # the same layer with per-(token, head) gates: KDA (b = w = beta) and
        # Gated DeltaNet (also a per-(token, head) decay).  The three are
        # timed interleaved, 3 rounds of 20 steps, and the medians reported;
        # GDN-2's time over KDA's is the measured cost of its two per-channel
        # gates.
        # A fourth entry, layer_prep, takes the raw layer inputs (q, k before
        # the L2 norm, b and w as logits, alpha as the float32 log-decay).
        beta = dev["b"][..., 0].contiguous()
        alpha_s = dev["alpha"][..., 0].contiguous()
        vins = {"gdn2": dev, "kda": dict(dev, b=beta, w=beta),
                "gated_deltanet": dict(dev, b=beta, w=beta, alpha=alpha_s),
                "layer_prep": dict(dev, alpha=torch.log(dev["alpha"].float()))}
        secs = {name: [] for name in vins}
        for _ in range(3):
            for name, vin in vins.items():
                secs[name].append(timed_steps(
                    lambda: g.chunk_fwd(*(vin[x] for x in NAMES), chunk=C, out=o, S_final=Sf, workspace=ws,
                                        path=args.path, layer_prep=(name == "layer_prep")), 20, 3))
        med = {name: float(np.median(v)) for name, v in secs.items()}
        variants = {name: {"tokens_per_s": round(B * T / t, 1), "ms": round(t * 1e3, 4)} for name, t in med.items()}
        variants["gdn2_over_kda_time"] = round(med["gdn2"] / med["kda"], 4)
        variants["gdn2_throughput_vs_gated_deltanet"] = round(med["gated_deltanet"] / med["gdn2"], 4)
        variants["layer_prep_over_gdn2_time"] = round(med["layer_prep"] / med["gdn2"], 4)
        out["gate_variants"] = variants
        del vins

        # token-by-token path (the cross-check and the R1 rule's GPU path) on
        # the first 1024 tokens of the same layer: rule R5 against rule R1
        Tr = 1024
        rin = {x: dev[x][:, :Tr].contiguous() for x in NAMES}
        orr = torch.empty((B, Tr, H, d), dtype=torch.bfloat16, device="cuda")
        rsec = {}
        for rule in ("R5", "R1"):
            rsec[rule] = timed_steps(lambda: g.chunk_fwd(*(rin[x] for x in NAMES), out=orr, S_final=Sf,
                                                         path="recurrent", rule=rule), 5, 1)
        out["token_recurrent"] = {
            "workload": f"B={B} T={Tr} H={H} d={d} bf16, token by token",
            "r5_tokens_per_s": round(B * Tr / rsec["R5"], 1), "r5_ms": round(rsec["R5"] * 1e3, 4),
            "r1_tokens_per_s": round(B * Tr / rsec["R1"], 1), "r1_ms": round(rsec["R1"] * 1e3, 4),
            "r1_over_r5_time": round(rsec["R1"] / rsec["R5"], 4),
        }
        del rin, orr

        # rule R1 on the chunked two-pass path, the same layer
        ws_r1 = torch.empty(g.workspace_bytes(B, T, H, d, d, 0, C, torch.bfloat16, g.FLAG_RULE_R1),
                            dtype=torch.uint8, device="cuda")
        g.profile_enable(True)
        g.profile_read(reset=True)
        sec_r1 = timed_steps(lambda: g.chunk_fwd(*(dev[x] for x in NAMES), chunk=C, out=o, S_final=Sf,
                                                 workspace=ws_r1, rule="R1"), 20, 5)
        r1prof = g.profile_read(reset=True)
        g.profile_enable(False)
        out["rule_r1_chunked"] = {
            "workload": "the same layer (8 x 4096 x 16 heads, d=128, bf16), rule R1, two-pass kernels",
            "tokens_per_s": round(B * T / sec_r1, 1), "ms": round(sec_r1 * 1e3, 4),
            "r1_over_r5_time": round(sec_r1 / sec, 4),
            "kernels": {k: {"avg_us": 1e3 * ms / n, "launches": n} for k, (ms, n) in r1prof.items()},
        }
        del ws_r1

        lens = gi.packed_lengths(3)
        cu = gi.cu_seqlens_from(lens).cuda()
        packed = {x: dev[x].view(1, 32768, H, d) for x in NAMES}
        Sp = torch.empty((len(lens), H, d, d), dtype=torch.float32, device="cuda")
        wsp = torch.empty(g.workspace_bytes(1, 32768, H, d, d, len(lens), C, torch.bfloat16),
                          dtype=torch.uint8, device="cuda")
        sec_p = timed_steps(lambda: g.chunk_fwd(*(packed[x] for x in NAMES), cu_seqlens=cu,
                                                chunk=C, out=o.view(1, 32768, H, d), S_final=Sp,
                                                workspace=wsp, path=args.path), 20, 3)
        out["packed"] = {"tokens_per_s": round(32768 / sec_p, 1), "num_seqs": len(lens),
                         "ms": round(sec_p * 1e3, 4)}

        # decode: 256 sequences x 16 heads, 16 distinct step inputs cycled
        c4 = gi.WORKLOADS["decode_256x16_d128"]
        dd = gi.make_decode_inputs(c4["N"], c4["H"], d, d, "bf16", c4["seed"], steps=c4["steps"])
        ddev = {x: dd[x].cuda() for x in NAMES}
        S_a = dd["S"].cuda()
        S_b = dd["S"].cuda().clone()
        od = torch.empty((c4["N"], c4["H"], d), dtype=torch.bfloat16, device="cuda")
        step_bytes = c4["N"] * c4["H"] * (2 * d * d * 4 + 7 * d * 2)
        counter = [0]

        def dstep(states):
            i = counter[0]
            counter[0] += 1
            g.decode_step(*(ddev[x][i % c4["steps"]] for x in NAMES), states[i % len(states)],
                          out=od)

        # eager launches, no timing hooks
        sec_d = timed_steps(lambda: dstep([S_a]), args.decode_steps, 10)
        # the same loop as HIP graph replays: one graph of c4["steps"]
        # consecutive steps (each distinct input once, the state in place)
        gsteps = c4["steps"]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for t in range(gsteps):
                g.decode_step(*(ddev[x][t] for x in NAMES), S_a, out=od)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        dgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(dgraph):
            for t in range(gsteps):
                g.decode_step(*(ddev[x][t] for x in NAMES), S_a, out=od)
        replays = max(1, args.decode_steps // gsteps)
        sec_dg = timed_steps(dgraph.replay, replays, 2) / gsteps
        del dgraph
        # kernel durations: HIP events around every launch, in passes of their own
        hooked = max(100, args.decode_steps // 5)
        g.profile_enable(True)
        timed_steps(lambda: dstep([S_a]), hooked, 10)
        dprof = g.profile_read(reset=True)
        timed_steps(lambda: dstep([S_a, S_b]), hooked, 10)
        dprof_c = g.profile_read(reset=True)
        g.profile_enable(False)
        dk_us = 1e3 * dprof["decode"][0] / dprof["decode"][1]
        dkc_us = 1e3 * dprof_c["decode"][0] / dprof_c["decode"][1]
        out["decode"] = {
            "workload": "256 sequences x 16 heads, d=128, bf16 inputs, fp32 state in place",
            "steps": args.decode_steps, "us_per_step": round(sec_d * 1e6, 2),
            "graph_us_per_step": round(sec_dg * 1e6, 2),
            "graph": f"{replays} replays of one HIP graph of {gsteps} consecutive steps",
            "kernel_us": round(dk_us, 2),
            "algorithmic_bytes_per_step": step_bytes,
            "GBps": round(step_bytes / (dk_us * 1e-6) / 1e9, 1),
            "hbm_frac": round(step_bytes / (dk_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "oracle_ms_per_step": None,
            "two_state_buffers": {"kernel_us": round(dkc_us, 2),
                                  "GBps": round(step_bytes / (dkc_us * 1e-6) / 1e9, 1),
                                  "hbm_frac": round(step_bytes / (dkc_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        }

        if not args.no_cpu:
            # the oracle's decode step on the same state and inputs, all host
            # threads over the 4096 (sequence, head) units, 20 steps
            import oracle
            S_host = dd["S"].double().numpy()
            t0 = time.perf_counter()
            for i in range(20):
                _, S_host = oracle.decode(*(dd[x][i % c4["steps"]] for x in NAMES), S_host)
            out["decode"]["oracle_ms_per_step"] = round((time.perf_counter() - t0) / 20 * 1e3, 2)
            out["decode"]["oracle_cores"] = oracle.max_threads()
            del S_host

        # the chunked backward of the same layer (dL/do ~ N(0,1), dL/dS_final = 0)
        grads = gi.make_bwd_grads(B, T, H, d, d, "bf16", seed=2, with_dS=False)
        dout = grads["dout"].cuda()
        wsb = torch.empty(g.bwd_workspace_bytes(B, T, H, d, d, 0, C, torch.bfloat16), dtype=torch.uint8,
                          device="cuda")
        gout = {n: torch.empty_like(dev[x]) for n, x in zip(("dq", "dk", "dv", "dalpha", "db", "dw"), NAMES)}
        gout["dS0"] = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda")

        def bstep():
            g.chunk_bwd(*(dev[x] for x in NAMES), dout, chunk=C, workspace=wsb, out=gout)

        del ws
        bstep()
        torch.cuda.synchronize()
        g.profile_enable(True)
        g.profile_read(reset=True)
        bsteps = max(3, args.steps // 5)
        sec_b = timed_steps(bstep, bsteps, 2)
        bprof = g.profile_read(reset=True)
        g.profile_enable(False)
        bkern = {k: {"avg_us": 1e3 * ms / n, "launches": n} for k, (ms, n) in bprof.items()}
        # the same backward for KDA inputs (b = w = beta per (token, head))
        kin = dict(dev, b=dev["b"][..., 0].contiguous(), w=dev["b"][..., 0].contiguous())
        kout = dict(gout, db=torch.empty_like(kin["b"]), dw=torch.empty_like(kin["w"]))
        sec_bk = timed_steps(lambda: g.chunk_bwd(*(kin[x] for x in NAMES), dout, chunk=C, workspace=wsb, out=kout),
                             bsteps, 2)
        # a training step: the forward (two-pass path) into the backward's
        # workspace, then the backward with the forward's blocks handed over
        o_t = torch.empty_like(o)
        Sf_t = torch.empty_like(Sf)

        def fwd_into_wsb():
            g.chunk_fwd(*(dev[x] for x in NAMES), chunk=C, out=o_t, S_final=Sf_t, workspace=wsb, path="two_pass")

        def bstep_prepared():
            g.chunk_bwd(*(dev[x] for x in NAMES), dout, chunk=C, workspace=wsb, out=gout, prepared=True)

        def train_step():
            fwd_into_wsb()
            bstep_prepared()

        sec_train = timed_steps(train_step, bsteps, 2)
        fwd_into_wsb()
        sec_bp = timed_steps(bstep_prepared, bsteps, 2)

        # the same with the states kept by the forward's scan (the backward
        # skips its states scan too)
        def train_step_kept():
            g.chunk_fwd(*(dev[x] for x in NAMES), chunk=C, out=o_t, S_final=Sf_t, workspace=wsb, path="two_pass",
                        keep_states=True)
            g.chunk_bwd(*(dev[x] for x in NAMES), dout, chunk=C, workspace=wsb, out=gout, prepared=True,
                        states_kept=True)

        sec_train_kept = timed_steps(train_step_kept, bsteps, 2)
        bbyt = bwd_bytes_per_token_head(d, C)
        bdom = max(bkern, key=lambda k: bkern[k]["avg_us"])
        bach = bbyt[bdom] * tok_heads / (bkern[bdom]["avg_us"] * 1e-6) / 1e9
        out["backward"] = {
            "workload": "gdn2_chunk_bwd of the same layer: dq, dk, dv, dalpha, db, dw, dS0",
            "steps": bsteps, "ms_per_step": round(sec_b * 1e3, 4),
            "tokens_per_s": round(B * T / sec_b, 1),
            "time_over_forward": round(sec_b / sec, 3),
            "kda_ms_per_step": round(sec_bk * 1e3, 4),
            "gdn2_over_kda_time": round(sec_b / sec_bk, 4),
            "prepared_ms_per_step": round(sec_bp * 1e3, 4),
            "train_step": {"workload": "forward (two-pass) into the backward's workspace, then the backward "
                                       "with the forward's per-chunk blocks handed over",
                           "ms_per_step": round(sec_train * 1e3, 4),
                           "tokens_per_s": round(B * T / sec_train, 1),
                           "states_kept_ms_per_step": round(sec_train_kept * 1e3, 4)},
            "path_algorithmic_bytes": int(bbyt["path"] * tok_heads),
            "path_hbm_frac": round(bbyt["path"] * tok_heads / sec_b / 1e9 / HBM_PEAK_GBS, 4),
            "kernels": bkern,
            "roofline": {"bound": "hbm", "kernel": bdom, "achieved": round(bach, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(bach / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes_per_launch": int(bbyt[bdom] * tok_heads)},
        }
        del wsb

        out["context_parallel"] = context_parallel(g, dev, H, d, C, args.path)

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp, H, args.cpu_budget)
        if args.configs:
            out["configs"] = configs_table(g)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out))
    return 0


if __name__ == "__main__":
    sys.exit(main())
