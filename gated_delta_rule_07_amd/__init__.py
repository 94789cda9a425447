"""Python binding of libgdn2, the MI355X (gfx950) hot path (forward, backward,
decode) of the Gated DeltaNet-2 recurrence.

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libgdn2.so`` (built in-tree by ``gated_delta_rule_07_amd.build``).
PyTorch provides device memory and the current HIP stream.  There is no CPU
fallback: without the library or a GPU these functions raise.

    o, S_final = chunk_fwd(q, k, v, alpha, b, w, S0=None, cu_seqlens=None, chunk=64)
    grads = chunk_bwd(q, k, v, alpha, b, w, dout, S0=None, dS_final=None, ...)
    o = decode_step(q, k, v, alpha, b, w, S)      # S updated in place
    Phi, Psi = segment_map(q, k, v, alpha, b, w)  # per-sequence state maps
    S_in, S_final = segment_combine(Phi, Psi, S0) # entering state of each segment

Shapes: q, k, alpha, b [B, T, H, dk]; v, w [B, T, H, dv] (packed sequences:
B = 1 and ``cu_seqlens`` int32 [N + 1] on the device); states [N, H, dk, dv]
float32.  Inputs are float32 or bfloat16 and must all have the same dtype.
In ``chunk_fwd``, b, w and alpha may instead be [B, T, H] (one value per
token and head, shared by its channels): b = w = beta is KDA, with a
[B, T, H] alpha too it is Gated DeltaNet.  With ``layer_prep=True`` the
inputs are the raw layer projections: q, k not normalised, b and w logits,
and alpha the float32 natural-log decay (float32 whatever the other dtype).
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn2.so")

GDN2_F32, GDN2_BF16 = 0, 1
FLAG_RECURRENT = 1 << 1
FLAG_TWO_PASS = 1 << 2
FLAG_FUSED = 1 << 3
FLAG_SCALAR_B = 1 << 4
FLAG_SCALAR_W = 1 << 5
FLAG_SCALAR_ALPHA = 1 << 6
FLAG_LAYER_PREP = 1 << 0
FLAG_RULE_R1 = 1 << 7
FLAG_PREPARED = 1 << 8
FLAG_KEEP_STATES = 1 << 9
PATHS = {"auto": 0, "recurrent": FLAG_RECURRENT, "two_pass": FLAG_TWO_PASS, "fused": FLAG_FUSED}
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP error"}

_lib = None


class Gdn2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libgdn2: {STATUS.get(status, status)}: {msg}")
        self.status = status


def configure(L: ctypes.CDLL) -> ctypes.CDLL:
    """Sets the argument and result types of every C-ABI entry point on a
    loaded copy of the library and returns it."""
    vp, i, sz, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint32
    L.gdn2_chunk_fwd_workspace_bytes.restype = sz
    L.gdn2_chunk_fwd_workspace_bytes.argtypes = [i] * 7 + [i]
    L.gdn2_chunk_fwd_workspace_bytes_flags.restype = sz
    L.gdn2_chunk_fwd_workspace_bytes_flags.argtypes = [i] * 7 + [i, u32]
    L.gdn2_chunk_fwd.restype = i
    L.gdn2_chunk_fwd.argtypes = [vp] * 8 + [i] * 8 + [u32, vp, vp, vp, sz, vp]
    L.gdn2_chunk_fwd_noalloc.restype = i
    L.gdn2_chunk_fwd_noalloc.argtypes = [vp] * 8 + [i] * 8 + [u32, vp, vp, vp]
    L.gdn2_chunk_bwd_workspace_bytes.restype = sz
    L.gdn2_chunk_bwd_workspace_bytes.argtypes = [i] * 7 + [i]
    L.gdn2_chunk_bwd.restype = i
    L.gdn2_chunk_bwd.argtypes = [vp] * 8 + [i] * 8 + [u32] + [vp] * 9 + [vp, sz, vp]
    L.gdn2_chunk_segment_map.restype = i
    L.gdn2_chunk_segment_map.argtypes = [vp] * 7 + [i] * 8 + [u32, vp, vp, vp, sz, vp]
    L.gdn2_segment_combine.restype = i
    L.gdn2_segment_combine.argtypes = [vp] * 3 + [i] * 4 + [vp, vp, vp]
    L.gdn2_decode_step.restype = i
    L.gdn2_decode_step.argtypes = [vp] * 8 + [i] * 5 + [vp]
    L.gdn2_status_string.restype = ctypes.c_char_p
    L.gdn2_status_string.argtypes = [i]
    L.gdn2_last_error.restype = ctypes.c_char_p
    L.gdn2_last_error.argtypes = []
    L.gdn2_abi_version.restype = i
    L.gdn2_profile_enable.restype = i
    L.gdn2_profile_enable.argtypes = [i]
    L.gdn2_profile_read.restype = i
    L.gdn2_profile_read.argtypes = [i, ctypes.POINTER(ctypes.c_char_p),
                                    ctypes.POINTER(ctypes.c_double),
                                    ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int), i]
    return L


def lib() -> ctypes.CDLL:
    """The loaded ``libgdn2.so`` (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; run `python -m gated_delta_rule_07_amd.build`")
        _lib = configure(ctypes.CDLL(LIB_PATH))
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise Gdn2Error(status, lib().gdn2_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return GDN2_F32
    if t.dtype == torch.bfloat16:
        return GDN2_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _require_device(*ts) -> None:
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("libgdn2 takes contiguous device tensors")


def _require(t, name: str, shape: tuple, dtype) -> None:
    """A caller-provided tensor: on the device, contiguous, of this shape and dtype."""
    if t is None:
        return
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {list(shape)}, not {list(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, not {t.dtype}")


def _require_workspace(ws, need: int) -> int:
    """Bytes of a caller-provided workspace (a contiguous device tensor)."""
    if not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"workspace holds {nbytes} bytes, {need} are needed")
    return nbytes


def _gate_flags(q, v, alpha, b, w) -> int:
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    flags = 0
    for t, flag, name, full in ((b, FLAG_SCALAR_B, "b", dk), (w, FLAG_SCALAR_W, "w", dv),
                                (alpha, FLAG_SCALAR_ALPHA, "alpha", dk)):
        if tuple(t.shape) == (B, T, H):
            flags |= flag
        elif tuple(t.shape) != (B, T, H, full):
            raise ValueError(f"{name} must be [{B}, {T}, {H}, {full}] or [{B}, {T}, {H}]")
    return flags


def workspace_bytes(B: int, T: int, H: int, dk: int, dv: int, num_seqs: int, chunk: int,
                    dtype: torch.dtype, flags: int = 0) -> int:
    code = GDN2_BF16 if dtype == torch.bfloat16 else GDN2_F32
    return int(lib().gdn2_chunk_fwd_workspace_bytes_flags(B, T, H, dk, dv, num_seqs, chunk, code, flags))


def chunk_fwd(q, k, v, alpha, b, w, S0=None, cu_seqlens=None, chunk: int = 64,
              recurrent: bool = False, out=None, S_final=None, workspace=None,
              want_final: bool = True, path: str = "auto", layer_prep: bool = False,
              rule: str = "R5", prepared: bool = False, keep_states: bool = False):
    """Chunked forward.  ``path`` selects the kernels: "auto" (the library
    chooses), "fused" (single pass), "two_pass", or "recurrent" (token by
    token; also selected by ``recurrent=True``).  ``rule="R1"`` runs the
    alternative reading R1 (two-pass or token-by-token path).  ``prepared=True``
    runs the state scan alone on a ``workspace`` that ``segment_map`` (or a
    two-pass ``chunk_fwd``) filled for the same inputs.  ``keep_states=True``
    (two-pass path) also writes the state entering every chunk into a
    backward-sized ``workspace``, for ``chunk_bwd(..., prepared=True,
    states_kept=True)``.  Returns (o, S_final); S_final is None when
    ``want_final`` is False."""
    if recurrent:
        path = "recurrent"
    _require_device(q, k, v, alpha, b, w, S0, cu_seqlens)
    dt = _dtype_code(q)
    for t in (k, v, b, w) + (() if layer_prep else (alpha,)):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, alpha, b, w must share one dtype")
    if layer_prep and alpha.dtype != torch.float32:
        raise TypeError("with layer_prep, alpha is the float32 log-decay")
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q and v must be [B, T, H, d]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _require(k, "k", (B, T, H, dk), q.dtype)
    _require(v, "v", (B, T, H, dv), q.dtype)
    gate_flags = _gate_flags(q, v, alpha, b, w)
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
            raise TypeError("cu_seqlens must be a 1-D int32 tensor")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if S0 is not None and (S0.dtype != torch.float32 or tuple(S0.shape) != (N, H, dk, dv)):
        raise ValueError(f"S0 must be float32 [{N}, {H}, {dk}, {dv}]")
    _require(out, "out", (B, T, H, dv), q.dtype)
    _require(S_final, "S_final", (N, H, dk, dv), torch.float32)
    o = out if out is not None else torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    Sf = S_final
    if Sf is None and want_final:
        Sf = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    if rule not in ("R5", "R1"):
        raise ValueError(f"unknown rule {rule!r}")
    if prepared and workspace is None:
        raise ValueError("prepared=True reads the given workspace")
    flags = (PATHS[path] | gate_flags | (FLAG_LAYER_PREP if layer_prep else 0) | (FLAG_RULE_R1 if rule == "R1" else 0)
             | (FLAG_PREPARED if prepared else 0) | (FLAG_KEEP_STATES if keep_states else 0))
    ws_bytes = 0
    if path != "recurrent":
        ws_bytes = workspace_bytes(B, T, H, dk, dv, N if cu_seqlens is not None else 0, chunk, q.dtype, flags)
        if workspace is None:
            workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
            ws_bytes = workspace.numel()
        else:
            # a smaller workspace is allowed (the plain two-pass size): the library checks it
            ws_bytes = _require_workspace(workspace, 0)
    _check(lib().gdn2_chunk_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S0), _ptr(cu_seqlens),
        B, T, H, dk, dv, N if cu_seqlens is not None else 0, chunk, dt, flags,
        _ptr(o), _ptr(Sf), _ptr(workspace), ws_bytes, _stream()))
    return o, Sf


def bwd_workspace_bytes(B: int, T: int, H: int, dk: int, dv: int, num_seqs: int, chunk: int,
                        dtype: torch.dtype) -> int:
    code = GDN2_BF16 if dtype == torch.bfloat16 else GDN2_F32
    return int(lib().gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, dv, num_seqs, chunk, code))


def chunk_bwd(q, k, v, alpha, b, w, dout, S0=None, dS_final=None, cu_seqlens=None,
              chunk: int = 64, workspace=None, out=None, want_dS0: bool = True,
              layer_prep: bool = False, prepared: bool = False, states_kept: bool = False):
    """Chunked backward of ``chunk_fwd``, for the same input modes (b, w,
    alpha per channel or [B, T, H]; ``layer_prep`` for the raw layer
    inputs).  Given dL/do (``dout``, like o) and dL/dS_final (or None for
    zero), returns a dict with dq, dk, dv, dalpha, db, dw (each like its
    input: the gradient with respect to the input as given) and dS0
    ([N, H, dk, dv] float32, or None when ``want_dS0`` is False).  ``out``
    may hold preallocated tensors under those names.  ``prepared=True``
    takes the per-chunk blocks a ``chunk_fwd(..., path="two_pass")`` left in
    ``workspace`` (a backward-sized workspace, same inputs) instead of
    recomputing them; with ``states_kept=True`` as well, the states that a
    ``chunk_fwd(..., keep_states=True)`` kept there too."""
    _require_device(q, k, v, alpha, b, w, dout, S0, dS_final, cu_seqlens)
    dt = _dtype_code(q)
    for t in (k, v, b, w, dout) + (() if layer_prep else (alpha,)):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, alpha, b, w, dout must share one dtype")
    if layer_prep and alpha.dtype != torch.float32:
        raise TypeError("with layer_prep, alpha is the float32 log-decay")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    for t, name, full in ((k, "k", dk), (v, "v", dv), (dout, "dout", dv)):
        if tuple(t.shape) != (B, T, H, full):
            raise ValueError(f"{name} must be [{B}, {T}, {H}, {full}]")
    flags = (_gate_flags(q, v, alpha, b, w) | (FLAG_LAYER_PREP if layer_prep else 0)
             | (FLAG_PREPARED if prepared else 0) | (FLAG_KEEP_STATES if states_kept else 0))
    if prepared and workspace is None:
        raise ValueError("prepared=True reads the given workspace")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    for t, name in ((S0, "S0"), (dS_final, "dS_final")):
        if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != (N, H, dk, dv)):
            raise ValueError(f"{name} must be float32 [{N}, {H}, {dk}, {dv}]")
    out = dict(out or {})
    src = {"dq": q, "dk": k, "dv": v, "dalpha": alpha, "db": b, "dw": w}
    for name, like in src.items():
        if name not in out:
            out[name] = torch.empty_like(like)
    if want_dS0 and "dS0" not in out:
        out["dS0"] = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    ns = N if cu_seqlens is not None else 0
    ws_bytes = bwd_workspace_bytes(B, T, H, dk, dv, ns, chunk, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    for name, like in src.items():
        _require(out[name], name, tuple(like.shape), like.dtype)
    _require(out.get("dS0"), "dS0", (N, H, dk, dv), torch.float32)
    _check(lib().gdn2_chunk_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(S0), _ptr(cu_seqlens),
        B, T, H, dk, dv, ns, chunk, dt, flags, _ptr(dout), _ptr(dS_final),
        _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dalpha"]), _ptr(out["db"]),
        _ptr(out["dw"]), _ptr(out.get("dS0")), _ptr(workspace), _require_workspace(workspace, 0), _stream()))
    out.setdefault("dS0", None)
    return out


def segment_map(q, k, v, alpha, b, w, cu_seqlens=None, chunk: int = 64, layer_prep: bool = False,
                workspace=None, out=None):
    """Affine state map of every sequence of the call (each taken as one
    segment of a longer sequence): returns (Phi [N, H, dk, dk], Psi
    [N, H, dk, dv]) float32 with S_out = Phi S_in + Psi.  Inputs as for
    ``chunk_fwd`` (gate layouts and ``layer_prep`` included).  ``out`` may
    be a preallocated (Phi, Psi) pair."""
    _require_device(q, k, v, alpha, b, w, cu_seqlens)
    dt = _dtype_code(q)
    for t in (k, v, b, w) + (() if layer_prep else (alpha,)):
        if t.dtype != q.dtype:
            raise TypeError("q, k, v, alpha, b, w must share one dtype")
    if layer_prep and alpha.dtype != torch.float32:
        raise TypeError("with layer_prep, alpha is the float32 log-decay")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    flags = _gate_flags(q, v, alpha, b, w) | (FLAG_LAYER_PREP if layer_prep else 0)
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if out is not None:
        Phi, Psi = out
    else:
        Phi = torch.empty((N, H, dk, dk), dtype=torch.float32, device=q.device)
        Psi = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    _require_device(Phi, Psi)
    if tuple(Phi.shape) != (N, H, dk, dk) or tuple(Psi.shape) != (N, H, dk, dv) or \
            Phi.dtype != torch.float32 or Psi.dtype != torch.float32:
        raise ValueError(f"Phi, Psi must be float32 [{N}, {H}, {dk}, {dk}] and [{N}, {H}, {dk}, {dv}]")
    ns = N if cu_seqlens is not None else 0
    ws_bytes = workspace_bytes(B, T, H, dk, dv, ns, chunk, q.dtype)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    _check(lib().gdn2_chunk_segment_map(
        _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w), _ptr(cu_seqlens),
        B, T, H, dk, dv, ns, chunk, dt, flags, _ptr(Phi), _ptr(Psi), _ptr(workspace),
        _require_workspace(workspace, 0), _stream()))
    return Phi, Psi


def segment_combine(Phi, Psi, S0=None, want_final: bool = True, out=None):
    """Exclusive scan of the maps of G consecutive segments of one sequence
    (Phi [G, H, dk, dk], Psi [G, H, dk, dv]) from S0 [H, dk, dv] (None: zero).
    Returns (S_in [G, H, dk, dv], S_final [H, dk, dv] or None)."""
    _require_device(Phi, Psi, S0)
    G, H, dk, _ = Phi.shape
    dv = Psi.shape[-1]
    if Phi.dtype != torch.float32 or Psi.dtype != torch.float32 or tuple(Psi.shape) != (G, H, dk, dv):
        raise ValueError("Phi, Psi must be float32 [G, H, dk, dk] and [G, H, dk, dv]")
    if S0 is not None and (S0.dtype != torch.float32 or tuple(S0.shape) != (H, dk, dv)):
        raise ValueError(f"S0 must be float32 [{H}, {dk}, {dv}]")
    S_in = out if out is not None else torch.empty((G, H, dk, dv), dtype=torch.float32, device=Phi.device)
    Sf = torch.empty((H, dk, dv), dtype=torch.float32, device=Phi.device) if want_final else None
    _check(lib().gdn2_segment_combine(_ptr(Phi), _ptr(Psi), _ptr(S0), G, H, dk, dv, _ptr(S_in), _ptr(Sf),
                                      _stream()))
    return S_in, Sf


def decode_step(q, k, v, alpha, b, w, S, out=None):
    """One decode step: inputs [N, H, d]; S [N, H, dk, dv] float32, updated in place."""
    _require_device(q, k, v, alpha, b, w, S)
    dt = _dtype_code(q)
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q and v must be [N, H, d]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    for t, name, d in ((k, "k", dk), (alpha, "alpha", dk), (b, "b", dk), (v, "v", dv), (w, "w", dv)):
        _require(t, name, (N, H, d), q.dtype)
    if S.dtype != torch.float32 or tuple(S.shape) != (N, H, dk, dv):
        raise ValueError(f"S must be float32 [{N}, {H}, {dk}, {dv}]")
    _require(out, "out", (N, H, dv), q.dtype)
    o = out if out is not None else torch.empty((N, H, dv), dtype=q.dtype, device=q.device)
    _check(lib().gdn2_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(b), _ptr(w),
                                  _ptr(S), _ptr(o), N, H, dk, dv, dt, _stream()))
    return o


def profile_enable(on: bool = True) -> None:
    _check(lib().gdn2_profile_enable(1 if on else 0))


def profile_read(reset: bool = True) -> dict:
    """{kernel name: (total ms, launches)} since the last reset."""
    n = ctypes.c_int(0)
    cap = 16
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_double * cap)()
    cnt = (ctypes.c_int * cap)()
    _check(lib().gdn2_profile_read(cap, names, ms, cnt, ctypes.byref(n), 1 if reset else 0))
    return {names[i].decode(): (ms[i], cnt[i]) for i in range(min(n.value, cap))}
