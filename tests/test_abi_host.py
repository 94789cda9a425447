"""Host-side checks of libgdn2 that need no GPU: the library loads, exports
every function include/gdn2.h declares, and rejects bad arguments with the
documented status before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn2.h")


# Every host-side check runs against the product library and against its
# host-checked build (the C-ABI layer with undefined-behaviour checks that
# trap: an overflow in the size arithmetic or an out-of-bounds host access
# ends the test process instead of passing silently).
@pytest.fixture(scope="module", params=["libgdn2.so", "libgdn2_hostcheck.so"])
def L(request):
    import gated_delta_rule_07_amd as g
    if request.param == "libgdn2.so":
        if not os.path.exists(g.LIB_PATH):
            pytest.fail("libgdn2.so is not built (run __graft_entry__.build())")
        return g.lib()
    path = os.path.join(os.path.dirname(g.LIB_PATH), request.param)
    if not os.path.exists(path):
        pytest.fail(f"{request.param} is not built (run __graft_entry__.build())")
    return g.configure(ctypes.CDLL(path))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn2_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), f"{n} declared in gdn2.h but not exported"


def test_abi_version_and_status_strings(L):
    assert L.gdn2_abi_version() == 1
    assert L.gdn2_status_string(0) == b"ok"
    assert L.gdn2_status_string(3) == b"workspace too small"
    assert L.gdn2_status_string(99) == b"unknown status"


F32, BF16 = 0, 1
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every case fails validation first


def call_fwd(L, *, ptr=FAKE, B=1, T=64, H=1, dk=16, dv=16, N=0, chunk=16, dt=F32, flags=0,
             cu=None, ws=FAKE, ws_bytes=1 << 40, S0=None, q=None):
    p = ptr
    return L.gdn2_chunk_fwd(q if q is not None else p, p, p, p, p, p, S0, cu, B, T, H, dk, dv, N,
                            chunk, dt, flags, p, None, ws, ws_bytes, None)


def test_fwd_rejects_before_launch(L):
    assert call_fwd(L, dk=24, dv=24) == 2
    assert call_fwd(L, dk=64, dv=48) == 2
    assert call_fwd(L, dk=16, dv=64, ws_bytes=100) == 3   # dk != dv widens in the workspace: size-checked first
    assert call_fwd(L, chunk=32) == 2
    assert call_fwd(L, dt=7) == 2
    assert call_fwd(L, B=0) == 1
    assert call_fwd(L, T=-1) == 1
    assert call_fwd(L, flags=1 << 10) == 1         # unknown flag
    # kept states: two-pass path of rule R5, square heads, backward-sized workspace
    for other in (1 << 1, 1 << 3, 1 << 7):
        assert call_fwd(L, flags=(1 << 9) | other) == 2
    assert call_fwd(L, flags=1 << 9, dk=16, dv=32) == 2
    fwd_ws = L.gdn2_chunk_fwd_workspace_bytes(1, 64, 1, 16, 16, 0, 16, F32)
    assert call_fwd(L, flags=1 << 9, ws_bytes=fwd_ws) == 3   # room for the blocks, not the states
    assert call_fwd(L, flags=(1 << 8) | (1 << 1)) == 2         # prepared workspace on the token-by-token path
    assert call_fwd(L, flags=(1 << 8) | (1 << 3)) == 2         # prepared workspace on the single-pass path
    assert call_fwd(L, flags=1 << 8, ws_bytes=100) == 3        # a prepared workspace is still size-checked
    assert call_fwd(L, flags=(1 << 7) | (1 << 3)) == 2         # rule R1 has no single-pass kernel
    assert call_fwd(L, flags=(1 << 7) | (1 << 8)) == 2         # nor a prepared workspace
    assert call_fwd(L, flags=1 << 7, dk=128, dv=128, chunk=64) == 2   # float32, d = 128, chunk 64: not built
    assert call_fwd(L, flags=1 << 7, ws_bytes=100) == 3        # its larger blocks are size-checked
    assert call_fwd(L, flags=(1 << 2) | (1 << 3)) == 1         # two paths at once
    assert call_fwd(L, flags=(1 << 1) | (1 << 4)) == 2         # token-by-token path with a per-(token, head) gate
    assert call_fwd(L, flags=(1 << 1) | (1 << 6)) == 2
    assert call_fwd(L, flags=(1 << 1) | (1 << 0)) == 2         # token-by-token path with layer prep
    assert call_fwd(L, ptr=0) == 1
    assert call_fwd(L, q=FAKE + 4) == 1                       # misaligned
    assert call_fwd(L, N=3) == 1                              # num_seqs without cu_seqlens
    assert call_fwd(L, cu=FAKE, B=2, N=2) == 1                # packed needs B == 1
    assert call_fwd(L, cu=FAKE, N=0) == 1                     # packed needs num_seqs
    assert call_fwd(L, ws_bytes=100) == 3
    assert b"workspace" in L.gdn2_last_error()
    assert call_fwd(L, ws=0) == 3


def test_workspace_bytes(L):
    f = L.gdn2_chunk_fwd_workspace_bytes
    # the layer workload: 8 x 64 chunks x 16 heads of bf16 intermediates, 70 KiB
    # each: -W, Q', Kbar^T (16 KiB each), gamma_C and P's 10 tiles (to 54 KiB
    # in whole KiB), Ut (16 KiB); in front of them the 256-byte chunk table
    w = f(8, 4096, 16, 128, 128, 0, 64, BF16)
    assert w == 256 + 8 * 64 * 16 * 70 * 1024
    assert f(8, 4096, 16, 128, 64, 0, 64, BF16) > w   # dk != dv: the square call plus the widened copies
    assert f(1, 100, 2, 64, 64, 5, 16, F32) >= f(1, 100, 2, 64, 64, 0, 16, F32)


def test_workspace_bytes_long_sequence(L):
    # B sequences of 128 chunks or more with at most 32 (sequence, head)
    # units also reserve the segment schedule: G = min(16, 128 / (B H),
    # chunks / 16) segments per sequence (packed: the mean length), their
    # bounds, chunk table, blocks of the packed layout, and Phi, Psi, S_in.
    # Shorter sequences and more units get the plain size.
    d, C = 128, 64

    def ws(B, T, H, n=0):
        return L.gdn2_chunk_fwd_workspace_bytes(B, T, H, d, d, n, C, BF16)

    blk = (ws(1, C, 1) - 256) // 2          # one chunk slot of one head (B = 1 reserves nc + 1 slots)
    assert blk > 0 and ws(1, C, 1) == 256 + 2 * blk

    def plain(B, T, H, n=0):
        nc = -(-T // C)
        m = n if n > 0 else B
        return 256 * (-(-(m + 1) * 4 // 256)) + max(B * nc, nc + m) * H * blk

    def seg(B, T, H, G, total=None):
        # B sequences of T tokens (or `total` tokens in all, packed), G segments each
        nt = -(-(total if total is not None else B * T) // C)
        blocks = (nt + B * G) * H * blk
        return 2 * 256 * (-(-(B * G + 1) * 4 // 256)) + -(-blocks // 256) * 256 + 3 * B * G * H * d * d * 4

    assert ws(1, 32768, 16) == max(plain(1, 32768, 16), seg(1, 32768, 16, 8))
    assert ws(1, 32768, 16) > plain(1, 32768, 16)
    assert ws(1, 40000, 3) == max(plain(1, 40000, 3), seg(1, 40000, 3, 16))      # 625 chunks, 3 heads
    assert ws(1, 128 * C, 16) == max(plain(1, 128 * C, 16), seg(1, 128 * C, 16, 8))
    assert ws(1, 256 * C, 8) == max(plain(1, 256 * C, 8), seg(1, 256 * C, 8, 16))
    assert ws(2, 256 * C, 8) == max(plain(2, 256 * C, 8), seg(2, 256 * C, 8, 8))  # 16 (sequence, head) units
    assert ws(4, 200 * C, 2) == max(plain(4, 200 * C, 2), seg(4, 200 * C, 2, 8))
    assert ws(1, 127 * C, 16) == plain(1, 127 * C, 16)       # 127 chunks
    assert ws(2, 32768, 16) == max(plain(2, 32768, 16), seg(2, 32768, 16, 4))   # 32 units
    assert ws(1, 32768, 17) == max(plain(1, 32768, 17), seg(1, 32768, 17, 4))   # 17 heads
    assert ws(1, 32768, 33) == plain(1, 32768, 33)           # 33 units
    assert ws(3, 32768, 11) == plain(3, 32768, 11)           # 33 units
    assert ws(1, 32768, 16, 1) == max(plain(1, 32768, 16), seg(1, 32768, 16, 8))   # one packed sequence
    assert ws(1, 32768, 8, 2) == max(plain(1, 32768, 8, 2), seg(2, 16384, 8, 8))   # two, 256 chunks on average
    assert ws(1, 32768, 16, 2) == max(plain(1, 32768, 16, 2), seg(2, 16384, 16, 4))   # 32 units
    assert ws(1, 32768, 11, 3) == plain(1, 32768, 11, 3)     # 33 units
    assert ws(1, 32768, 4, 3) == max(plain(1, 32768, 4, 3), seg(3, 0, 4, 8, total=32768))


def test_decode_rejects_before_launch(L):
    p = FAKE
    assert L.gdn2_decode_step(p, p, p, p, p, p, p, p, 4, 2, 16, 16, 5, None) == 2
    assert L.gdn2_decode_step(p, p, p, p, p, p, p, p, 0, 2, 16, 16, 0, None) == 1
    assert L.gdn2_decode_step(p, p, p, p, p, p, None, p, 4, 2, 16, 16, 0, None) == 1
    assert L.gdn2_decode_step(p, p, p, p, p, p, p, p, 4, 2, 48, 48, 0, None) == 2


def test_profile_read_empty(L):
    n = ctypes.c_int(-1)
    assert L.gdn2_profile_read(0, None, None, None, ctypes.byref(n), 1) == 0
    assert n.value == 0


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "use.c"
    src.write_text('#include "gdn2.h"\nint main(void){ return gdn2_abi_version() == 0; }\n')
    import subprocess
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only",
                        "-I", os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def call_bwd(L, *, ptr=FAKE, B=1, T=64, H=1, dk=16, dv=16, N=0, chunk=16, dt=F32, flags=0,
             cu=None, ws=FAKE, ws_bytes=1 << 40, dout=None, dq=None):
    p = ptr
    return L.gdn2_chunk_bwd(p, p, p, p, p, p, None, cu, B, T, H, dk, dv, N, chunk, dt, flags,
                            dout if dout is not None else p, None, dq if dq is not None else p,
                            p, p, p, p, p, None, ws, ws_bytes, None)


def test_bwd_rejects_before_launch(L):
    assert call_bwd(L, dk=24, dv=24) == 2
    assert call_bwd(L, dk=64, dv=48) == 2
    assert call_bwd(L, chunk=32) == 2
    assert call_bwd(L, dt=7) == 2
    assert call_bwd(L, B=0) == 1
    assert call_bwd(L, T=-1) == 1
    # the backward takes no forward path or rule flag, nor kept states
    # without the forward's blocks
    for flag in (1 << 1, 1 << 2, 1 << 3, 1 << 7, 1 << 9, 1 << 10):
        assert call_bwd(L, flags=flag) == 2
    assert call_bwd(L, flags=(1 << 8) | (1 << 9), ws_bytes=16) == 3
    # the forward's blocks handed over: square heads only, still size-checked
    assert call_bwd(L, flags=1 << 8, dk=16, dv=32) == 2
    assert call_bwd(L, flags=1 << 8, ws_bytes=16) == 3
    assert call_bwd(L, dout=0x10008) == 1      # misaligned
    assert call_bwd(L, ws_bytes=16) == 3
    assert call_bwd(L, B=2, N=1) == 1          # num_seqs without cu_seqlens
    assert call_bwd(L, B=2, N=2, cu=FAKE) == 1  # packed needs B == 1
    assert L.gdn2_last_error() != b""


def test_bwd_workspace_bytes(L):
    n = L.gdn2_chunk_bwd_workspace_bytes(2, 200, 3, 64, 64, 0, 64, BF16)
    fwd = L.gdn2_chunk_fwd_workspace_bytes(2, 200, 3, 64, 64, 0, 64, BF16)
    # the forward's blocks (its workspace less the chunk table) plus the
    # entering state and the leaving-state gradient of every chunk-head
    # (2 sequences x 4 chunks x 3 heads), each a set of bfloat16 tiles
    assert n >= fwd - 256 + 2 * (2 * 4 * 3) * 64 * 64 * 2
    assert L.gdn2_chunk_bwd_workspace_bytes(2, 200, 3, 48, 48, 0, 64, BF16) == 0
    assert L.gdn2_chunk_bwd_workspace_bytes(1, 300, 2, 32, 32, 3, 16, F32) >= \
        L.gdn2_chunk_bwd_workspace_bytes(1, 300, 2, 32, 32, 0, 16, F32)


def call_segmap(L, *, ptr=FAKE, B=1, T=64, H=1, dk=16, dv=16, N=0, chunk=16, dt=F32, flags=0,
                cu=None, ws=FAKE, ws_bytes=1 << 40, phi=FAKE, psi=FAKE):
    p = ptr
    return L.gdn2_chunk_segment_map(p, p, p, p, p, p, cu, B, T, H, dk, dv, N, chunk, dt, flags,
                                    phi, psi, ws, ws_bytes, None)


def test_segment_map_rejects_before_launch(L):
    assert call_segmap(L, dk=24, dv=24) == 2
    assert call_segmap(L, dk=64, dv=32) == 2
    assert call_segmap(L, chunk=32) == 2
    assert call_segmap(L, dt=7) == 2
    assert call_segmap(L, B=0) == 1
    assert call_segmap(L, T=-1) == 1
    # path and rule flags do not apply to the map
    for flag in (1 << 1, 1 << 2, 1 << 3, 1 << 7, 1 << 8, 1 << 9):
        assert call_segmap(L, flags=flag) == 2
    assert call_segmap(L, phi=None) == 1
    assert call_segmap(L, psi=0x10004) == 1      # misaligned
    assert call_segmap(L, ws_bytes=16) == 3
    assert call_segmap(L, B=2, N=1) == 1         # num_seqs without cu_seqlens
    assert call_segmap(L, B=2, N=2, cu=FAKE) == 1
    assert L.gdn2_last_error() != b""


def test_segment_combine_rejects_before_launch(L):
    p = FAKE
    assert L.gdn2_segment_combine(p, p, None, -1, 1, 16, 16, p, None, None) == 1
    assert L.gdn2_segment_combine(p, p, None, 2, 0, 16, 16, p, None, None) == 1
    assert L.gdn2_segment_combine(p, p, None, 2, 1, 48, 48, p, None, None) == 2
    assert L.gdn2_segment_combine(p, p, None, 2, 1, 32, 16, p, None, None) == 2
    assert L.gdn2_segment_combine(None, p, None, 2, 1, 16, 16, p, None, None) == 1
    assert L.gdn2_segment_combine(p, p, None, 2, 1, 16, 16, None, None, None) == 1
    assert L.gdn2_segment_combine(p, p, 0x10008, 2, 1, 16, 16, p, None, None) == 1
    # nothing to do: no segment and no final state asked for
    assert L.gdn2_segment_combine(None, None, None, 0, 1, 16, 16, None, None, None) == 0


def call_noalloc(L, *, ptr=FAKE, B=1, T=64, H=1, dk=16, dv=16, N=0, chunk=16, dt=F32, flags=0, cu=None):
    p = ptr
    return L.gdn2_chunk_fwd_noalloc(p, p, p, p, p, p, None, cu, B, T, H, dk, dv, N, chunk, dt, flags, p, None, None)


def test_noalloc_rejects_before_launch(L):
    """The allocation-free forward checks its arguments before it touches the
    device: path, rule and prepared-workspace flags, sizes, null pointers,
    and packed input larger than its scratch."""
    for flag in (1 << 1, 1 << 3, 1 << 7, 1 << 8, 1 << 9):
        assert call_noalloc(L, flags=flag) == 2
    assert call_noalloc(L, dk=24, dv=24) == 2
    assert call_noalloc(L, chunk=32) == 2
    assert call_noalloc(L, dt=7) == 2
    assert call_noalloc(L, B=0) == 1
    assert call_noalloc(L, ptr=0) == 1
    assert call_noalloc(L, cu=FAKE, N=0) == 1
    # 1 x 65536 packed tokens x 16 heads, d = 128: far more than the scratch
    assert call_noalloc(L, cu=FAKE, N=4, T=65536, H=16, dk=128, dv=128, chunk=64, dt=BF16) == 3
    assert b"scratch" in L.gdn2_last_error()


def test_workspace_bytes_rule_r1(L):
    f = L.gdn2_chunk_fwd_workspace_bytes
    fl = L.gdn2_chunk_fwd_workspace_bytes_flags
    L.gdn2_chunk_fwd_workspace_bytes_flags.argtypes = [ctypes.c_int] * 8 + [ctypes.c_uint32]
    L.gdn2_chunk_fwd_workspace_bytes_flags.restype = ctypes.c_size_t
    assert fl(8, 4096, 16, 128, 128, 0, 64, BF16, 0) == f(8, 4096, 16, 128, 128, 0, 64, BF16)
    # rule R1: per chunk-head -W', Q'', Ebar^T, gamma_C, -Ut', O'' and N (dk x dv, bf16): over 32 KiB more
    r1 = fl(8, 4096, 16, 128, 128, 0, 64, BF16, 1 << 7)
    assert r1 >= f(8, 4096, 16, 128, 128, 0, 64, BF16) + 8 * 64 * 16 * 32 * 1024 - 4096
    assert fl(1, 100, 2, 128, 128, 0, 64, F32, 1 << 7) == 0      # not built
    assert fl(1, 100, 2, 128, 128, 0, 16, F32, 1 << 7) > 0


def test_sizes_at_the_limits(L):
    """Workspace sizes and argument checks with sizes near the int range:
    every product is formed in size_t, so nothing overflows (the host-checked
    build traps on a signed overflow), and calls the library cannot serve
    are refused or sized as 0, never wrapped around."""
    f, fb = L.gdn2_chunk_fwd_workspace_bytes, L.gdn2_chunk_bwd_workspace_bytes
    big = 2 ** 31 - 1
    for B, T, H in ((1, big, 1), (big, 64, 1), (1, 64, big), (2 ** 16, 2 ** 16, 16), (1, big, 64)):
        for dt in (F32, BF16):
            w = f(B, T, H, 128, 128, 0, 64, dt)
            assert w == 0 or w >= B * H * ((T + 63) // 64) * 1024
            wb = fb(B, T, H, 128, 128, 0, 64, dt)
            assert wb == 0 or wb >= w
    # the limits: chunk slots x heads below 2^24, sequences x heads at most
    # 2^21, inputs at most 2^40 elements; past them the size is 0
    assert f(1, 2 ** 24, 16, 64, 64, 2 ** 16, 64, BF16) > 0
    assert f(1, 2 ** 24, 16, 64, 64, 2 ** 18, 64, BF16) == 0      # 2^22 sequence-heads
    assert f(1, 2 ** 26, 16, 128, 128, 0, 64, BF16) == 0          # 2^24 chunk-heads
    assert f(1, 2 ** 26 - 64, 16, 128, 128, 0, 64, BF16) > 0
    assert f(1, 1, 1, 16, 16, big, 16, F32) == 0
    # the entry points refuse such sizes before touching a pointer
    assert call_fwd(L, B=big, T=big, H=big, ws_bytes=1 << 40) == 2
    assert call_fwd(L, T=big, H=big, ws_bytes=1 << 40) == 2
    assert call_fwd(L, B=1, T=2 ** 26, H=16, dk=128, dv=128, chunk=64, ws_bytes=1 << 50) == 2


def test_workspace_bytes_rectangular_heads(L):
    """dk != dv: the square call's workspace on d = max(dk, dv) plus the
    widened copies of the narrower side and one d x d state per
    (sequence, head), each rounded up to 256 bytes."""
    f, fb = L.gdn2_chunk_fwd_workspace_bytes, L.gdn2_chunk_bwd_workspace_bytes
    for dk, dv in ((16, 64), (64, 16), (128, 64), (32, 128)):
        d = max(dk, dv)
        for B, T, H, n, C, dt in ((2, 200, 3, 0, 64, BF16), (1, 300, 4, 3, 16, F32)):
            sq = f(B, T, H, d, d, n, C, dt)
            slot = -(-B * T * H * d * 4 // 256) * 256
            N = n if n > 0 else B
            state = -(-N * H * d * d * 4 // 256) * 256
            assert f(B, T, H, dk, dv, n, C, dt) == sq + (4 if dk < d else 3) * slot + state
            # the backward: an input and a gradient slot for each of the
            # narrower side's tensors (q, k, alpha, b or v, w, plus dout),
            # and three states: S0, dL/dS_final, dL/dS0
            sqb = fb(B, T, H, d, d, n, C, dt)
            assert fb(B, T, H, dk, dv, n, C, dt) == sqb + (8 if dk < d else 5) * slot + 3 * state
    assert f(2, 64, 2, 16, 48, 0, 64, BF16) == 0
    assert fb(2, 64, 2, 16, 48, 0, 64, BF16) == 0


def test_keep_states_workspace_bytes(L):
    """With kept states the forward needs the backward's workspace (square
    heads only)."""
    f = L.gdn2_chunk_fwd_workspace_bytes_flags
    f.restype = ctypes.c_size_t
    for args in ((2, 200, 3, 64, 64, 0, 64, BF16), (1, 300, 2, 32, 32, 3, 16, F32)):
        assert f(*args, 1 << 9) == L.gdn2_chunk_bwd_workspace_bytes(*args) > L.gdn2_chunk_fwd_workspace_bytes(*args)
    assert f(2, 200, 3, 64, 32, 0, 64, BF16, 1 << 9) == 0
