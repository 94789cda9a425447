// gdn2_api.cpp -- the C ABI of libgdn2 (include/gdn2.h): argument checks,
// workspace planning, kernel selection and launches on the caller's stream.
// No memory is allocated and the stream is never synchronised.
#include "../../include/gdn2.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "gdn2_kernels.hpp"

namespace {

thread_local std::string g_last_error;

gdn2_status_t fail(gdn2_status_t st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

gdn2_status_t ok() {
  g_last_error.clear();
  return GDN2_OK;
}

bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool supported_chunk(int c) { return c == 16 || c == 64; }

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// ------------------------------------------------------------- profiling --
// Kernel names are string literals of this file, so the pointers handed out
// by gdn2_profile_read stay valid for the life of the library.
struct prof_rec {
  const char *name;
  hipEvent_t start, stop;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<prof_rec> g_prof_pending;
std::vector<std::pair<const char *, std::pair<double, int>>> g_prof_total;

struct prof_scope {
  hipStream_t st;
  bool on;
  prof_rec rec;
  prof_scope(const char *name, hipStream_t s) : st(s), on(false) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!g_prof_on)
      return;
    // no system-scope fence: a fenced event would write back the L2 between
    // the two passes and slow down the very launches being timed
    if (hipEventCreateWithFlags(&rec.start, hipEventDisableSystemFence) != hipSuccess)
      return;
    if (hipEventCreateWithFlags(&rec.stop, hipEventDisableSystemFence) != hipSuccess) {
      (void)hipEventDestroy(rec.start);
      return;
    }
    rec.name = name;
    on = hipEventRecord(rec.start, st) == hipSuccess;
    if (!on) {
      (void)hipEventDestroy(rec.start);
      (void)hipEventDestroy(rec.stop);
    }
  }
  ~prof_scope() {
    if (!on)
      return;
    (void)hipEventRecord(rec.stop, st);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_pending.push_back(rec);
  }
};

// --------------------------------------------------------------- dispatch --
template <typename IO, int D, int C> size_t block_bytes() { return gdn2::chunk_block_bytes<IO, D, C>(); }

size_t chunk_block_bytes_rt(gdn2_dtype_t dt, int d, int c) {
#define GDN2_BB(IO, D, C) \
  if (d == D && c == C)   \
    return block_bytes<IO, D, C>();
  if (dt == GDN2_F32) {
    GDN2_BB(float, 16, 16) GDN2_BB(float, 32, 16) GDN2_BB(float, 64, 16) GDN2_BB(float, 128, 16)
    GDN2_BB(float, 16, 64) GDN2_BB(float, 32, 64) GDN2_BB(float, 64, 64) GDN2_BB(float, 128, 64)
  } else {
    GDN2_BB(gdn2::bf16_t, 16, 16) GDN2_BB(gdn2::bf16_t, 32, 16) GDN2_BB(gdn2::bf16_t, 64, 16)
    GDN2_BB(gdn2::bf16_t, 128, 16) GDN2_BB(gdn2::bf16_t, 16, 64) GDN2_BB(gdn2::bf16_t, 32, 64)
    GDN2_BB(gdn2::bf16_t, 64, 64) GDN2_BB(gdn2::bf16_t, 128, 64)
  }
#undef GDN2_BB
  return 0;
}

size_t r1_block_bytes_rt(gdn2_dtype_t dt, int d, int c) {
#define GDN2_RB1(IO, D, C) \
  if (d == D && c == C)    \
    return gdn2::r1_block_bytes<IO, D, C>();
  if (dt == GDN2_F32) {
    GDN2_RB1(float, 16, 16) GDN2_RB1(float, 32, 16) GDN2_RB1(float, 64, 16) GDN2_RB1(float, 128, 16)
    GDN2_RB1(float, 16, 64) GDN2_RB1(float, 32, 64) GDN2_RB1(float, 64, 64)
  } else {
    GDN2_RB1(gdn2::bf16_t, 16, 16) GDN2_RB1(gdn2::bf16_t, 32, 16) GDN2_RB1(gdn2::bf16_t, 64, 16)
    GDN2_RB1(gdn2::bf16_t, 128, 16) GDN2_RB1(gdn2::bf16_t, 16, 64) GDN2_RB1(gdn2::bf16_t, 32, 64)
    GDN2_RB1(gdn2::bf16_t, 64, 64) GDN2_RB1(gdn2::bf16_t, 128, 64)
  }
#undef GDN2_RB1
  return 0;  // float32 with d = 128 and chunk 64: not built (its LDS does not fit)
}

// Rule R1 on the two-pass path: chunk table (packed input), its per-chunk
// kernel, its state scan.
template <typename IO, int D, int C>
hipError_t run_chunk_r1(const gdn2::chunk_args &a, int C_rt, hipStream_t st) {
  hipError_t e = hipSuccess;
  if (a.cu) {
    prof_scope p("chunk_table", st);
    e = gdn2::launch_chunk_table(a.cu, a.num_seqs, C_rt, a.offsets, st);
    if (e != hipSuccess)
      return e;
  }
  {
    prof_scope p("r1_prep", st);
    e = gdn2::launch_r1_prep<IO, D, C>(a, st);
    if (e != hipSuccess)
      return e;
  }
  prof_scope p("r1_scan", st);
  return gdn2::launch_r1_scan<IO, D, C>(a, st);
}

hipError_t dispatch_chunk_r1(gdn2_dtype_t dt, int d, int c, const gdn2::chunk_args &a, hipStream_t st) {
#define GDN2_RR1(IO, D, C) \
  if (d == D && c == C)    \
    return run_chunk_r1<IO, D, C>(a, C, st);
  if (dt == GDN2_F32) {
    GDN2_RR1(float, 16, 16) GDN2_RR1(float, 32, 16) GDN2_RR1(float, 64, 16) GDN2_RR1(float, 128, 16)
    GDN2_RR1(float, 16, 64) GDN2_RR1(float, 32, 64) GDN2_RR1(float, 64, 64)
  } else {
    GDN2_RR1(gdn2::bf16_t, 16, 16) GDN2_RR1(gdn2::bf16_t, 32, 16) GDN2_RR1(gdn2::bf16_t, 64, 16)
    GDN2_RR1(gdn2::bf16_t, 128, 16) GDN2_RR1(gdn2::bf16_t, 16, 64) GDN2_RR1(gdn2::bf16_t, 32, 64)
    GDN2_RR1(gdn2::bf16_t, 64, 64) GDN2_RR1(gdn2::bf16_t, 128, 64)
  }
#undef GDN2_RR1
  return hipErrorInvalidValue;
}

// Path choice for the chunked forward.  0 = two-pass, otherwise the column
// group count NG of the single-pass kernel.
template <typename IO, int D, int C> int choose_fused(long units, uint32_t flags) {
  const bool f1 = gdn2::fused_supported<IO, D, C, 1>();
  const bool f2 = gdn2::fused_supported<IO, D, C, 2>();
  if (flags & GDN2_FLAG_TWO_PASS)
    return 0;
  if (flags & GDN2_FLAG_FUSED)
    return (units >= 192 || !f2) ? (f1 ? 1 : -1) : 2;
  // Default: two-pass.  On MI355X the single-pass kernel is bound by the
  // serial latency of its per-chunk phases (one workgroup per head cannot hide
  // it), and measured slower than the two-pass kernels at every shape of the
  // benchmark (B*T = 32768, H = 16, d = 128), so it is opt-in.
  (void)units;
  return 0;
}

// table_ready: packed input whose chunk table is already in a.offsets (the
// segment schedule's last step, after its maps)
template <typename IO, int D, int C>
hipError_t run_chunk(const gdn2::chunk_args &a, int C_rt, uint32_t flags, hipStream_t st, bool table_ready) {
  hipError_t e = hipSuccess;
  const int ng = choose_fused<IO, D, C>(static_cast<long>(a.num_seqs) * a.H, flags);
  if (ng < 0)
    return hipErrorInvalidConfiguration;
  if (a.cu && !table_ready) {
    prof_scope p("chunk_table", st);
    e = gdn2::launch_chunk_table(a.cu, a.num_seqs, C_rt, a.offsets, st);
    if (e != hipSuccess)
      return e;
  }
  if (ng > 0) {
    prof_scope p("chunk_fused", st);
    return ng == 1 ? gdn2::launch_fused<IO, D, C, 1>(a, st) : gdn2::launch_fused<IO, D, C, 2>(a, st);
  }
  if (!(flags & GDN2_FLAG_PREPARED)) {
    prof_scope p("chunk_prep", st);
    e = gdn2::launch_chunk_prep<IO, D, C>(a, st);
    if (e != hipSuccess)
      return e;
  }
  {
    prof_scope p("chunk_scan", st);
    e = (flags & GDN2_FLAG_KEEP_STATES) ? gdn2::launch_chunk_scan_keep<IO, D, C>(a, st)
                                        : gdn2::launch_chunk_scan<IO, D, C>(a, st);
  }
  return e;
}

hipError_t dispatch_chunk(gdn2_dtype_t dt, int d, int c, const gdn2::chunk_args &a, uint32_t flags,
                          hipStream_t st, bool table_ready = false) {
#define GDN2_RC(IO, D, C) \
  if (d == D && c == C)   \
    return run_chunk<IO, D, C>(a, C, flags, st, table_ready);
  if (dt == GDN2_F32) {
    GDN2_RC(float, 16, 16) GDN2_RC(float, 32, 16) GDN2_RC(float, 64, 16) GDN2_RC(float, 128, 16)
    GDN2_RC(float, 16, 64) GDN2_RC(float, 32, 64) GDN2_RC(float, 64, 64) GDN2_RC(float, 128, 64)
  } else {
    GDN2_RC(gdn2::bf16_t, 16, 16) GDN2_RC(gdn2::bf16_t, 32, 16) GDN2_RC(gdn2::bf16_t, 64, 16)
    GDN2_RC(gdn2::bf16_t, 128, 16) GDN2_RC(gdn2::bf16_t, 16, 64) GDN2_RC(gdn2::bf16_t, 32, 64)
    GDN2_RC(gdn2::bf16_t, 64, 64) GDN2_RC(gdn2::bf16_t, 128, 64)
  }
#undef GDN2_RC
  return hipErrorInvalidValue;
}

bool fused_available(gdn2_dtype_t dt, int d, int c) {
#define GDN2_FA(IO, D, C) \
  if (d == D && c == C)   \
    return gdn2::fused_supported<IO, D, C, 1>();
  if (dt == GDN2_F32) {
    GDN2_FA(float, 16, 16) GDN2_FA(float, 32, 16) GDN2_FA(float, 64, 16) GDN2_FA(float, 128, 16)
    GDN2_FA(float, 16, 64) GDN2_FA(float, 32, 64) GDN2_FA(float, 64, 64) GDN2_FA(float, 128, 64)
  } else {
    GDN2_FA(gdn2::bf16_t, 16, 16) GDN2_FA(gdn2::bf16_t, 32, 16) GDN2_FA(gdn2::bf16_t, 64, 16)
    GDN2_FA(gdn2::bf16_t, 128, 16) GDN2_FA(gdn2::bf16_t, 16, 64) GDN2_FA(gdn2::bf16_t, 32, 64)
    GDN2_FA(gdn2::bf16_t, 64, 64) GDN2_FA(gdn2::bf16_t, 128, 64)
  }
#undef GDN2_FA
  return false;
}

hipError_t dispatch_recurrent(gdn2_dtype_t dt, int dk, int dv, const void *q, const void *k, const void *v,
                              const void *al, const void *b, const void *w, const float *S0,
                              const int32_t *cu, int T, int H, int N, void *o, float *Sf, bool r1,
                              hipStream_t st) {
  prof_scope p("recurrent", st);
#define GDN2_RR(IO, DK, DV) \
  if (dk == DK && dv == DV) \
    return gdn2::launch_recurrent<IO, DK, DV>(q, k, v, al, b, w, S0, cu, T, H, N, o, Sf, r1, st);
#define GDN2_RR_DK(IO, DK) GDN2_RR(IO, DK, 16) GDN2_RR(IO, DK, 32) GDN2_RR(IO, DK, 64) GDN2_RR(IO, DK, 128)
  if (dt == GDN2_F32) {
    GDN2_RR_DK(float, 16) GDN2_RR_DK(float, 32) GDN2_RR_DK(float, 64) GDN2_RR_DK(float, 128)
  } else {
    GDN2_RR_DK(gdn2::bf16_t, 16) GDN2_RR_DK(gdn2::bf16_t, 32) GDN2_RR_DK(gdn2::bf16_t, 64)
    GDN2_RR_DK(gdn2::bf16_t, 128)
  }
#undef GDN2_RR_DK
#undef GDN2_RR
  return hipErrorInvalidValue;
}

hipError_t dispatch_decode(gdn2_dtype_t dt, int dk, int dv, const void *q, const void *k, const void *v,
                           const void *al, const void *b, const void *w, float *S, void *o, int N,
                           int H, hipStream_t st) {
  prof_scope p("decode", st);
#define GDN2_DD(IO, DK, DV) \
  if (dk == DK && dv == DV) \
    return gdn2::launch_decode<IO, DK, DV>(q, k, v, al, b, w, S, o, N, H, st);
#define GDN2_DD_DK(IO, DK) GDN2_DD(IO, DK, 16) GDN2_DD(IO, DK, 32) GDN2_DD(IO, DK, 64) GDN2_DD(IO, DK, 128)
  if (dt == GDN2_F32) {
    GDN2_DD_DK(float, 16) GDN2_DD_DK(float, 32) GDN2_DD_DK(float, 64) GDN2_DD_DK(float, 128)
  } else {
    GDN2_DD_DK(gdn2::bf16_t, 16) GDN2_DD_DK(gdn2::bf16_t, 32) GDN2_DD_DK(gdn2::bf16_t, 64)
    GDN2_DD_DK(gdn2::bf16_t, 128)
  }
#undef GDN2_DD_DK
#undef GDN2_DD
  return hipErrorInvalidValue;
}

// Chunk slots of a call: ceil(T / C) per sequence, or for packed input an
// upper bound of the sum of ceil(len / C).  Formed in 64 bits; every entry
// point checks sizes_supported first, so a call's count fits an int.
long long num_slots_for(int B, int T, int num_seqs, int chunk, bool packed) {
  const long long per = (static_cast<long long>(T) + chunk - 1) / chunk;
  return packed ? per + num_seqs : static_cast<long long>(B) * per;
}

// The sizes the library serves.  A dispatch holds its grid size in 32-bit
// work-item counts: the per-chunk kernels launch one workgroup of up to 256
// threads per chunk-head, so chunk slots x heads stay below 2^24; the scans
// launch up to two workgroups of up to 576 threads per (sequence, head), so
// sequences x heads stay at or below 2^21.  The inputs hold at most 2^40
// elements.
constexpr long long kMaxChunkHeads = (1LL << 24) - 1;
constexpr long long kMaxSeqHeads = 1LL << 21;

bool sizes_supported(int B, int T, int H, int d, int num_seqs, int chunk, bool packed) {
  if (B <= 0 || T < 0 || H <= 0 || d <= 0 || chunk <= 0 || num_seqs < 0 || (packed && num_seqs == 0))
    return false;
  const long long bt = static_cast<long long>(B) * T;
  if (bt > (1LL << 40) / (static_cast<long long>(H) * d))
    return false;
  const long long n = packed ? num_seqs : B;
  if (n > kMaxSeqHeads / H)
    return false;
  return num_slots_for(B, T, static_cast<int>(n), chunk, packed) <= kMaxChunkHeads / H;
}

// Calls with dk != dv run the chunked kernels on d = max(dk, dv) with the
// narrower side widened (gdn2_pad.hip says why that is exact).  In front of
// the widened call's own workspace: widened copies of the narrower side's
// inputs (q, k, alpha, b when dk < d; v, w and the widened o when dv < d),
// each slot sized for 4-byte elements (float32 inputs, or layer prep's
// float32 log-decay), and one d x d float32 state per (sequence, head) for
// S0 and S_final.
struct rect_plan {
  int d;
  size_t q, k, al, b, v, w, o, state, total;
};

rect_plan plan_rect(int B, int T, int H, int dk, int dv, int N) {
  rect_plan p{};
  p.d = dk > dv ? dk : dv;
  const size_t slot = align256(static_cast<size_t>(B) * T * H * p.d * 4);
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t at = off;
    off += n;
    return at;
  };
  if (dk < p.d) {
    p.q = take(slot);
    p.k = take(slot);
    p.al = take(slot);
    p.b = take(slot);
  }
  if (dv < p.d) {
    p.v = take(slot);
    p.w = take(slot);
    p.o = take(slot);
  }
  p.state = take(align256(static_cast<size_t>(N) * H * p.d * p.d * sizeof(float)));
  p.total = off;
  return p;
}

// The backward's widened call (dk != dv): slots for the narrower side's
// inputs and their gradients (q, k, alpha, b and dq, dk, dalpha, db when
// dk < d; v, w, dout and dv, dw when dv < d), then three d x d float32
// states per (sequence, head): S0, dL/dS_final and dL/dS0.
struct rect_bwd_plan {
  int d;
  size_t in[6], grad[6], dout, s0, dsf, ds0, total;  // in/grad index: q, k, v, alpha, b, w
};

rect_bwd_plan plan_rect_bwd(int B, int T, int H, int dk, int dv, int N) {
  rect_bwd_plan p{};
  p.d = dk > dv ? dk : dv;
  const size_t slot = align256(static_cast<size_t>(B) * T * H * p.d * 4);
  size_t off = 0;
  auto take = [&](size_t n) {
    const size_t at = off;
    off += n;
    return at;
  };
  const bool key_side[6] = {true, true, false, true, true, false};
  for (int i = 0; i < 6; ++i)
    if ((key_side[i] && dk < p.d) || (!key_side[i] && dv < p.d)) {
      p.in[i] = take(slot);
      p.grad[i] = take(slot);
    }
  if (dv < p.d)
    p.dout = take(slot);
  const size_t st = align256(static_cast<size_t>(N) * H * p.d * p.d * sizeof(float));
  p.s0 = take(st);
  p.dsf = take(st);
  p.ds0 = take(st);
  p.total = off;
  return p;
}

// ---------------------------------------------------------------- backward --
// The backward's share of the segment schedule (see run_segments): N
// sequences of T_total tokens in all, G segments each, and its workspace
// (bounds, chunk table, then Phi, Psi, S_in, Psi', X: [N, G, H, D, D]
// float32 each).
struct seg_run {
  char *ws;
  size_t cu_bytes;
  int N, G, T_total;
};

// Segment schedule of the backward.  The segments are whole chunks in
// order, so their chunk slots are numbered as the call's own: the blocks,
// states and state gradients land where the plain backward puts them (and
// a forward's blocks, with `prepared`, are read where it left them).
//   states: the segment maps from the prep's blocks, their scan from S0,
//     and the states-mode scan of every segment from its entering state;
//   state gradients: the reverse scan of every segment from zero gives
//     Psi'_g, the gradient of the state before segment g from g's own
//     outputs; the adjoint scan X(g - 1) = Phi_g^T X(g) + Psi'_g from
//     dL/dS_final gives the gradient after every segment (and dL/dS0); the
//     reverse scan of every segment from X(g) writes the final gradients.
// kept: a.states already holds the entering states (a forward's kept
// states); the maps are still needed for the state gradients
template <typename IO, int D, int C>
hipError_t run_bwd_segments(gdn2::bwd_args &ba, int C_rt, const seg_run &sg, bool prepared, bool kept,
                            hipStream_t st) {
  hipError_t e = hipSuccess;
  const gdn2::chunk_args &a = ba.f;
  const int nseg = sg.N * sg.G;
  const size_t mb = static_cast<size_t>(nseg) * a.H * D * D;
  int32_t *scu = reinterpret_cast<int32_t *>(sg.ws);
  int32_t *stab = reinterpret_cast<int32_t *>(sg.ws + sg.cu_bytes);
  float *Phi = reinterpret_cast<float *>(sg.ws + 2 * sg.cu_bytes);
  float *Psi = Phi + mb, *S_in = Psi + mb, *Psi2 = S_in + mb, *X = Psi2 + mb;
  gdn2::chunk_args s = a;
  s.cu = scu;
  s.offsets = stab;
  s.B = 1;
  s.T = sg.T_total;
  s.num_seqs = nseg;
  s.num_slots = static_cast<int>(num_slots_for(1, sg.T_total, nseg, C_rt, true));
  s.S0 = nullptr;
  s.S_final = nullptr;
  s.o = nullptr;
  {
    prof_scope p("segment_bounds", st);  // and their chunk table
    if ((e = gdn2::launch_seg_bounds(a.cu, scu, sg.G, a.T, sg.N, C_rt, st, stab)) != hipSuccess)
      return e;
  }
  if (!prepared) {
    prof_scope p("chunk_prep", st);
    if ((e = gdn2::launch_chunk_prep<IO, D, C>(s, st)) != hipSuccess)
      return e;
  }
  {
    prof_scope p("segment_map", st);
    if ((e = gdn2::launch_segmap<IO, D, C>(s, Phi, Psi, st)) != hipSuccess)
      return e;
  }
  if (!kept) {
    {
      prof_scope p("segment_combine", st);
      if ((e = gdn2::launch_seg_combine<D>(Phi, Psi, a.S0, sg.G, a.H, sg.N, S_in, nullptr, st, false)) !=
          hipSuccess)
        return e;
    }
    s.S0 = S_in;
    prof_scope p("chunk_states", st);
    if ((e = gdn2::launch_chunk_states<IO, D, C>(s, st)) != hipSuccess)
      return e;
  }
  gdn2::bwd_args bs = ba;
  bs.f = s;
  bs.dSf = nullptr;
  bs.dS0 = Psi2;
  {
    prof_scope p("bwd_dstate", st);
    if ((e = gdn2::launch_bwd_dstate<IO, D, C>(bs, st)) != hipSuccess)
      return e;
  }
  {
    prof_scope p("segment_combine", st);
    if ((e = gdn2::launch_seg_combine<D>(Phi, Psi2, ba.dSf, sg.G, a.H, sg.N, X, ba.dS0, st, true)) != hipSuccess)
      return e;
  }
  bs.dSf = X;
  bs.dS0 = nullptr;
  prof_scope p("bwd_dstate", st);
  return gdn2::launch_bwd_dstate<IO, D, C>(bs, st);
}

template <typename IO, int D, int C>
hipError_t run_bwd(gdn2::bwd_args &ba, int C_rt, const seg_run *sg, bool prepared, bool kept, hipStream_t st) {
  hipError_t e = hipSuccess;
  gdn2::chunk_args &a = ba.f;
  if (a.cu) {
    prof_scope p("chunk_table", st);
    e = gdn2::launch_chunk_table(a.cu, a.num_seqs, C_rt, a.offsets, st);
    if (e != hipSuccess)
      return e;
  }
  if (sg) {
    if ((e = run_bwd_segments<IO, D, C>(ba, C_rt, *sg, prepared, kept, st)) != hipSuccess)
      return e;
    prof_scope p("bwd_grad", st);
    return gdn2::launch_bwd_grad<IO, D, C>(ba, st);
  }
  if (a.num_slots > 0) {
    if (!prepared) {
      prof_scope p("chunk_prep", st);
      e = gdn2::launch_chunk_prep<IO, D, C>(a, st);
      if (e != hipSuccess)
        return e;
    }
    if (!kept) {
      prof_scope p("chunk_states", st);
      e = gdn2::launch_chunk_states<IO, D, C>(a, st);
      if (e != hipSuccess)
        return e;
    }
  }
  {
    prof_scope p("bwd_dstate", st);
    e = gdn2::launch_bwd_dstate<IO, D, C>(ba, st);
    if (e != hipSuccess)
      return e;
  }
  if (a.num_slots > 0) {
    prof_scope p("bwd_grad", st);
    e = gdn2::launch_bwd_grad<IO, D, C>(ba, st);
  }
  return e;
}

hipError_t dispatch_bwd(gdn2_dtype_t dt, int d, int c, gdn2::bwd_args &ba, const seg_run *sg, bool prepared,
                        bool kept, hipStream_t st) {
#define GDN2_RB(IO, D, C) \
  if (d == D && c == C)   \
    return run_bwd<IO, D, C>(ba, C, sg, prepared, kept, st);
  if (dt == GDN2_F32) {
    GDN2_RB(float, 16, 16) GDN2_RB(float, 32, 16) GDN2_RB(float, 64, 16) GDN2_RB(float, 128, 16)
    GDN2_RB(float, 16, 64) GDN2_RB(float, 32, 64) GDN2_RB(float, 64, 64) GDN2_RB(float, 128, 64)
  } else {
    GDN2_RB(gdn2::bf16_t, 16, 16) GDN2_RB(gdn2::bf16_t, 32, 16) GDN2_RB(gdn2::bf16_t, 64, 16)
    GDN2_RB(gdn2::bf16_t, 128, 16) GDN2_RB(gdn2::bf16_t, 16, 64) GDN2_RB(gdn2::bf16_t, 32, 64)
    GDN2_RB(gdn2::bf16_t, 64, 64) GDN2_RB(gdn2::bf16_t, 128, 64)
  }
#undef GDN2_RB
  return hipErrorInvalidValue;
}

// Byte layout of the backward's workspace: chunk table (packed input), the
// forward's per-chunk blocks, entering states, leaving-state gradients and
// one flag byte per chunk-head (strong decay: see gdn2_bwd_grad_kernel).
struct bwd_plan {
  size_t table, blocks, states, dstates, flags, total;
};

bwd_plan plan_bwd(gdn2_dtype_t dt, int B, int T, int H, int d, int N, int chunk, bool packed) {
  bwd_plan p{};
  const size_t slots = static_cast<size_t>(num_slots_for(B, T, N, chunk, packed));
  // a state as (d/16)^2 fragment tiles of the I/O type: one set (ColFrag)
  // for bfloat16, two (ColFrag, RowFrag) for float32
  const size_t sq = (dt == GDN2_BF16 ? 1 : 2) * static_cast<size_t>(d) * d * (dt == GDN2_BF16 ? 2 : 4);
  p.table = packed ? align256(static_cast<size_t>(N + 1) * sizeof(int32_t)) : 0;
  p.blocks = slots * H * chunk_block_bytes_rt(dt, d, chunk);
  p.states = align256(slots * H * sq);
  p.dstates = p.states;
  p.flags = align256(slots * H);  // one byte per chunk-head: the gradient kernel's strong-decay path
  p.total = p.table + p.blocks + p.states + p.dstates + p.flags;
  return p;
}


bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ------------------------------------------------------------ segment maps --
template <typename IO, int D, int C>
hipError_t run_segmap(const gdn2::chunk_args &a, int C_rt, float *Phi, float *Psi, hipStream_t st,
                      bool table_ready) {
  hipError_t e = hipSuccess;
  if (a.cu && !table_ready) {
    prof_scope p("chunk_table", st);
    e = gdn2::launch_chunk_table(a.cu, a.num_seqs, C_rt, a.offsets, st);
    if (e != hipSuccess)
      return e;
  }
  if (a.num_slots > 0) {
    prof_scope p("chunk_prep", st);
    e = gdn2::launch_chunk_prep<IO, D, C>(a, st);
    if (e != hipSuccess)
      return e;
  }
  prof_scope p("segment_map", st);
  return gdn2::launch_segmap<IO, D, C>(a, Phi, Psi, st);
}

hipError_t dispatch_segmap(gdn2_dtype_t dt, int d, int c, const gdn2::chunk_args &a, float *Phi, float *Psi,
                           hipStream_t st, bool table_ready = false) {
#define GDN2_RS(IO, D, C) \
  if (d == D && c == C)   \
    return run_segmap<IO, D, C>(a, C, Phi, Psi, st, table_ready);
  if (dt == GDN2_F32) {
    GDN2_RS(float, 16, 16) GDN2_RS(float, 32, 16) GDN2_RS(float, 64, 16) GDN2_RS(float, 128, 16)
    GDN2_RS(float, 16, 64) GDN2_RS(float, 32, 64) GDN2_RS(float, 64, 64) GDN2_RS(float, 128, 64)
  } else {
    GDN2_RS(gdn2::bf16_t, 16, 16) GDN2_RS(gdn2::bf16_t, 32, 16) GDN2_RS(gdn2::bf16_t, 64, 16)
    GDN2_RS(gdn2::bf16_t, 128, 16) GDN2_RS(gdn2::bf16_t, 16, 64) GDN2_RS(gdn2::bf16_t, 32, 64)
    GDN2_RS(gdn2::bf16_t, 64, 64) GDN2_RS(gdn2::bf16_t, 128, 64)
  }
#undef GDN2_RS
  return hipErrorInvalidValue;
}

// Segment-parallel schedule of the default forward for a few long
// sequences (fixed-length or packed).  With few (sequence, head) units the
// state scan, whose chunks run in order, occupies a fraction of the compute
// units.  Every sequence is then cut into G segments of whole chunks: their
// affine state maps (segment map kernel, on the prep's blocks; each
// sequence's last segment needs none), the exclusive scan of each sequence's
// maps from its S0, and the state scan of every segment from its entering
// state on the same blocks (the last segment's scan gives S_final).
// G = min(16, 128 / (N H), chunks / 16), with N sequences of (on average)
// `chunks` chunks, puts about 128 (segment, head) units on the GPU with
// segments of 16 chunks or more, for N H <= 32.  Measured on MI355X (bf16,
// d = 128, one sequence): 16 heads x 32768 tokens 0.71 ms against 0.89 ms
// for the serial scan, 16 x 16384 0.38 against 0.47, 8 x 16384 0.23 against
// 0.34, 4 x 8192 0.10 against 0.16, 4 x 65536 0.43 against 1.25; two
// sequences of 16384 x 16 heads (G = 4) 0.59 against 0.63.
int seg_count(int nc, int units) {
  int g = 16;
  while (g > 1 && (g * units > 128 || 16 * g > nc))
    g /= 2;
  return g;
}

// Sizes of a call as the schedule sees them: N sequences, T_total tokens in
// all, nc chunks per sequence (packed: the mean).
struct seg_shape {
  int N, T_total, nc;
};

seg_shape seg_shape_of(int B, int T, int num_seqs, int chunk, bool packed) {
  seg_shape x{};
  x.N = packed ? num_seqs : B;
  const long tt = packed ? static_cast<long>(T) : static_cast<long>(B) * T;
  x.T_total = tt > 0x7fffffffL ? -1 : static_cast<int>(tt);
  x.nc = x.N > 0 ? (packed ? static_cast<int>((tt + chunk - 1) / chunk / x.N) : (T + chunk - 1) / chunk) : 0;
  return x;
}

bool use_segments(const seg_shape &x, int H) {
  return x.N > 0 && x.T_total > 0 && static_cast<long>(x.N) * H <= 32 && x.nc >= 128 && seg_count(x.nc, x.N * H) >= 2;
}

struct seg_plan {
  size_t cu, table, blocks, map_bytes, total;
  int G;  // segments per sequence
};

seg_plan plan_segments(gdn2_dtype_t dt, const seg_shape &x, int H, int d, int chunk) {
  seg_plan p{};
  p.G = seg_count(x.nc, x.N * H);
  const int nseg = x.N * p.G;
  p.cu = align256(static_cast<size_t>(nseg + 1) * sizeof(int32_t));
  p.table = p.cu;
  p.blocks = align256(static_cast<size_t>(num_slots_for(1, x.T_total, nseg, chunk, true)) * H *
                      chunk_block_bytes_rt(dt, d, chunk));
  p.map_bytes = static_cast<size_t>(nseg) * H * d * d * sizeof(float);  // one of Phi, Psi, S_in
  p.total = p.cu + p.table + p.blocks + 3 * p.map_bytes;
  return p;
}

// Bytes the backward's segment schedule adds after the backward's own
// workspace: bounds and chunk table of N G segments, then Phi, Psi, S_in,
// Psi' and X.
size_t seg_bwd_extra(const seg_shape &x, int H, int d, size_t *cu_bytes = nullptr, int *G = nullptr) {
  const int g = seg_count(x.nc, x.N * H);
  const size_t cb = align256(static_cast<size_t>(x.N * g + 1) * sizeof(int32_t));
  if (cu_bytes)
    *cu_bytes = cb;
  if (G)
    *G = g;
  return 2 * cb + 5 * static_cast<size_t>(x.N) * g * H * d * d * sizeof(float);
}

hipError_t dispatch_combine(int d, const float *Phi, const float *Psi, const float *S0, int G, int H, int B,
                            float *S_in, float *S_final, hipStream_t st) {
  prof_scope p("segment_combine", st);
  switch (d) {
    case 16: return gdn2::launch_seg_combine<16>(Phi, Psi, S0, G, H, B, S_in, S_final, st);
    case 32: return gdn2::launch_seg_combine<32>(Phi, Psi, S0, G, H, B, S_in, S_final, st);
    case 64: return gdn2::launch_seg_combine<64>(Phi, Psi, S0, G, H, B, S_in, S_final, st);
    case 128: return gdn2::launch_seg_combine<128>(Phi, Psi, S0, G, H, B, S_in, S_final, st);
    default: return hipErrorInvalidValue;
  }
}

// The schedule above; `a` is the call's argument block (fixed-length or
// packed).  The N sequences are read as one packed stretch of tokens cut
// into N G segments, whose bounds a small kernel derives on the device.
hipError_t run_segments(gdn2_dtype_t dt, int d, int chunk, const gdn2::chunk_args &a, const seg_shape &x, char *ws,
                        hipStream_t st) {
  const seg_plan pl = plan_segments(dt, x, a.H, d, chunk);
  int32_t *cu = reinterpret_cast<int32_t *>(ws);
  float *Phi = reinterpret_cast<float *>(ws + pl.cu + pl.table + pl.blocks);
  float *Psi = Phi + pl.map_bytes / sizeof(float);
  float *S_in = Psi + pl.map_bytes / sizeof(float);
  hipError_t e = hipSuccess;
  {
    prof_scope p("segment_bounds", st);  // and their chunk table
    e = gdn2::launch_seg_bounds(a.cu, cu, pl.G, a.T, x.N, chunk, st, reinterpret_cast<int32_t *>(ws + pl.cu));
  }
  if (e != hipSuccess)
    return e;
  gdn2::chunk_args s = a;
  s.cu = cu;
  s.offsets = reinterpret_cast<int32_t *>(ws + pl.cu);
  s.B = 1;
  s.T = x.T_total;
  s.num_seqs = x.N * pl.G;
  s.num_slots = static_cast<int>(num_slots_for(1, s.T, s.num_seqs, chunk, true));
  s.blocks = ws + pl.cu + pl.table;
  s.S0 = nullptr;
  s.o = nullptr;
  s.S_final = nullptr;
  // the maps of every segment but each sequence's last, their scan from S0
  // (no S_final: the last segment's own state scan gives it), then every
  // segment's state scan from its entering state
  s.seg_G = pl.G;
  e = dispatch_segmap(dt, d, chunk, s, Phi, Psi, st, true);
  if (e != hipSuccess)
    return e;
  e = dispatch_combine(d, Phi, Psi, a.S0, pl.G, a.H, x.N, S_in, nullptr, st);
  if (e != hipSuccess)
    return e;
  s.S0 = S_in;
  s.o = a.o;
  s.S_final = a.S_final;
  return dispatch_chunk(dt, d, chunk, s, GDN2_FLAG_TWO_PASS | GDN2_FLAG_PREPARED, st, true);
}

// ------------------------------------------------------- no-alloc scratch --
// Device scratch of the allocation-free forward (gdn2_chunk_fwd_noalloc):
// one copy per GPU, reserved with the library's code object and held until
// the process ends.  In host code `scratch` is a host-side stand-in, not a
// device address: its address on a device comes from hipGetSymbolAddress,
// taken once per device with that device current, and only that address is
// passed to kernels.
static __device__ __align__(256) unsigned char scratch[GDN2_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (nullptr and a HIP error
// on failure).
void *device_scratch(hipError_t *err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess)
    return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    *err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !ptr) {
      if (*err == hipSuccess)
        *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t gdn2_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs, int chunk,
                                      gdn2_dtype_t dt) {
  if (B <= 0 || T < 0 || H <= 0 || !supported_dim(dk) || !supported_dim(dv) || !supported_chunk(chunk))
    return 0;
  if (dk != dv) {
    const int d = dk > dv ? dk : dv;
    const size_t inner = gdn2_chunk_fwd_workspace_bytes(B, T, H, d, d, num_seqs, chunk, dt);
    return inner == 0 ? 0 : plan_rect(B, T, H, dk, dv, num_seqs > 0 ? num_seqs : B).total + inner;
  }
  if (dt != GDN2_F32 && dt != GDN2_BF16)
    return 0;
  if (!sizes_supported(B, T, H, dk, B, chunk, false) ||
      (num_seqs > 0 && !sizes_supported(B, T, H, dk, num_seqs, chunk, true)))
    return 0;
  // num_seqs > 0 asks for packed input (B must then be 1); the bound returned
  // covers both the packed and the fixed-length layout of these sizes.
  const int n = num_seqs > 0 ? num_seqs : B;
  const size_t slots_fixed = static_cast<size_t>(num_slots_for(B, T, B, chunk, false));
  const size_t slots_packed = static_cast<size_t>(num_slots_for(B, T, n, chunk, true));
  const size_t slots = slots_packed > slots_fixed ? slots_packed : slots_fixed;
  const size_t table = align256(static_cast<size_t>(n + 1) * sizeof(int32_t));
  const size_t plain = table + slots * static_cast<size_t>(H) * chunk_block_bytes_rt(dt, dk, chunk);
  const seg_shape x = seg_shape_of(B, T, num_seqs, chunk, num_seqs > 0);
  if (use_segments(x, H)) {
    const size_t seg = plan_segments(dt, x, H, dk, chunk).total;
    return seg > plain ? seg : plain;
  }
  return plain;
}

size_t gdn2_chunk_fwd_workspace_bytes_flags(int B, int T, int H, int dk, int dv, int num_seqs, int chunk,
                                            gdn2_dtype_t dt, uint32_t flags) {
  if ((flags & GDN2_FLAG_KEEP_STATES) && !(flags & GDN2_FLAG_RECURRENT))
    return dk == dv ? gdn2_chunk_bwd_workspace_bytes(B, T, H, dk, dv, num_seqs, chunk, dt) : 0;
  if ((flags & GDN2_FLAG_RULE_R1) && !(flags & GDN2_FLAG_RECURRENT) && dk != dv) {
    if (!supported_dim(dk) || !supported_dim(dv))
      return 0;
    const int d = dk > dv ? dk : dv;
    const size_t inner = gdn2_chunk_fwd_workspace_bytes_flags(B, T, H, d, d, num_seqs, chunk, dt, flags);
    return inner == 0 ? 0 : plan_rect(B, T, H, dk, dv, num_seqs > 0 ? num_seqs : B).total + inner;
  }
  if ((flags & GDN2_FLAG_RULE_R1) && !(flags & GDN2_FLAG_RECURRENT)) {
    if (B <= 0 || T < 0 || H <= 0 || dk != dv || !supported_dim(dk) || !supported_chunk(chunk))
      return 0;
    if (dt != GDN2_F32 && dt != GDN2_BF16)
      return 0;
    if (!sizes_supported(B, T, H, dk, B, chunk, false) ||
        (num_seqs > 0 && !sizes_supported(B, T, H, dk, num_seqs, chunk, true)))
      return 0;
    const size_t blk = r1_block_bytes_rt(dt, dk, chunk);
    if (blk == 0)
      return 0;
    const int n = num_seqs > 0 ? num_seqs : B;
    const size_t slots_fixed = static_cast<size_t>(num_slots_for(B, T, B, chunk, false));
    const size_t slots_packed = static_cast<size_t>(num_slots_for(B, T, n, chunk, true));
    const size_t slots = slots_packed > slots_fixed ? slots_packed : slots_fixed;
    return align256(static_cast<size_t>(n + 1) * sizeof(int32_t)) + slots * static_cast<size_t>(H) * blk;
  }
  return gdn2_chunk_fwd_workspace_bytes(B, T, H, dk, dv, num_seqs, chunk, dt);
}

gdn2_status_t gdn2_chunk_fwd(const void *q, const void *k, const void *v, const void *alpha,
                             const void *b, const void *w, const float *S0,
                             const int32_t *cu_seqlens, int B, int T, int H, int dk, int dv,
                             int num_seqs, int chunk, gdn2_dtype_t dt, uint32_t flags, void *o,
                             float *S_final, void *workspace, size_t workspace_bytes,
                             void *stream) {
  if (dt != GDN2_F32 && dt != GDN2_BF16)
    return fail(GDN2_ERR_UNSUPPORTED, "gdn2_chunk_fwd: unknown dtype %d", static_cast<int>(dt));
  const uint32_t path_flags = GDN2_FLAG_RECURRENT | GDN2_FLAG_TWO_PASS | GDN2_FLAG_FUSED;
  const uint32_t gate_flags = GDN2_FLAG_SCALAR_B | GDN2_FLAG_SCALAR_W | GDN2_FLAG_SCALAR_ALPHA | GDN2_FLAG_LAYER_PREP;
  if (flags & ~(path_flags | gate_flags | GDN2_FLAG_RULE_R1 | GDN2_FLAG_PREPARED | GDN2_FLAG_KEEP_STATES))
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_fwd: unknown flags 0x%x", flags);
  const bool keep = (flags & GDN2_FLAG_KEEP_STATES) != 0;
  if (keep) {
    if (flags & (GDN2_FLAG_RECURRENT | GDN2_FLAG_FUSED | GDN2_FLAG_RULE_R1))
      return fail(GDN2_ERR_UNSUPPORTED, "gdn2_chunk_fwd: states are kept by the two-pass path of rule R5 only");
    if (dk != dv)
      return fail(GDN2_ERR_UNSUPPORTED,
                  "gdn2_chunk_fwd: GDN2_FLAG_KEEP_STATES needs dk == dv (the backward's workspace layout)");
    flags |= GDN2_FLAG_TWO_PASS;
  }
  if (flags & GDN2_FLAG_PREPARED) {
    if (flags & (GDN2_FLAG_RECURRENT | GDN2_FLAG_FUSED))
      return fail(GDN2_ERR_UNSUPPORTED, "gdn2_chunk_fwd: a prepared workspace is read by the two-pass path only");
    flags |= GDN2_FLAG_TWO_PASS;
  }
  const bool r1_chunked = (flags & GDN2_FLAG_RULE_R1) && !(flags & GDN2_FLAG_RECURRENT);
  if (r1_chunked && (flags & (GDN2_FLAG_FUSED | GDN2_FLAG_PREPARED)))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_fwd: rule R1 runs on the two-pass and token-by-token paths (no single-pass kernel, "
                "no prepared workspace)");
  {
    const uint32_t paths = flags & path_flags;
    if (paths & (paths - 1))
      return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_fwd: flags 0x%x name more than one path", flags);
  }
  if ((flags & GDN2_FLAG_RECURRENT) && (flags & gate_flags))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_fwd: the token-by-token path takes neither per-(token, head) gates nor layer prep");
  if (B <= 0 || T < 0 || H <= 0)
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_fwd: bad sizes B=%d T=%d H=%d", B, T, H);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_fwd: unsupported head dims dk=%d dv=%d (need dk, dv in {16,32,64,128})", dk, dv);
  if (!supported_chunk(chunk))
    return fail(GDN2_ERR_UNSUPPORTED, "gdn2_chunk_fwd: unsupported chunk %d (need 16 or 64)", chunk);
  const bool packed = cu_seqlens != nullptr;
  int N;
  if (packed) {
    if (B != 1)
      return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_fwd: packed input needs B == 1 (got %d)", B);
    if (num_seqs <= 0)
      return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_fwd: packed input needs num_seqs > 0");
    N = num_seqs;
  } else {
    if (num_seqs != 0 && num_seqs != B)
      return fail(GDN2_ERR_INVALID_ARGUMENT,
                  "gdn2_chunk_fwd: num_seqs=%d must be 0 or B=%d without cu_seqlens", num_seqs, B);
    N = B;
  }
  if (T > 0 && (!q || !k || !v || !alpha || !b || !w || !o))
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_fwd: null input or output pointer");
  const void *ptrs[] = {q, k, v, alpha, b, w, S0, o, S_final, workspace};
  for (const void *p : ptrs)
    if (p && !aligned16(p))
      return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_fwd: pointers must be 16-byte aligned");
  if (!sizes_supported(B, T, H, dk > dv ? dk : dv, N, chunk, packed))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_fwd: sizes beyond the library's limits (at most 2^40 input elements, 2^24 chunk-heads, "
                "2^21 sequence-heads)");
  hipStream_t st = static_cast<hipStream_t>(stream);

  if (flags & GDN2_FLAG_RECURRENT) {
    const hipError_t e = dispatch_recurrent(dt, dk, dv, q, k, v, alpha, b, w, S0, cu_seqlens, T, H, N,
                                            o, S_final, (flags & GDN2_FLAG_RULE_R1) != 0, st);
    if (e != hipSuccess)
      return fail(GDN2_ERR_HIP, "gdn2_chunk_fwd: launch failed: %s", hipGetErrorString(e));
    return ok();
  }

  if (dk != dv) {
    // the chunked kernels on d = max(dk, dv), the narrower side widened in
    // the front of the workspace, o and S_final narrowed back afterwards
    const rect_plan rp = plan_rect(B, T, H, dk, dv, N);
    const int d = rp.d;
    if (workspace_bytes < rp.total || !workspace)
      return fail(GDN2_ERR_WORKSPACE_TOO_SMALL,
                  "gdn2_chunk_fwd: workspace of %zu bytes is smaller than the %zu needed to widen dk=%d dv=%d to %d",
                  workspace_bytes, rp.total, dk, dv, d);
    char *wsr = static_cast<char *>(workspace);
    const long long rows = static_cast<long long>(B) * T * H;
    const int E = dt == GDN2_BF16 ? 2 : 4;
    const uint32_t one_bits = dt == GDN2_BF16 ? 0x3F80u : 0x3F800000u;  // 1.0: no decay
    hipError_t e = hipSuccess;
    auto widen = [&](const void *src, size_t at, int width, int esz, uint32_t fill) -> const void * {
      if (e == hipSuccess)
        e = gdn2::launch_pad(src, wsr + at, rows, 1, width, 1, d, esz, fill, st);
      return wsr + at;
    };
    const void *q2 = q, *k2 = k, *al2 = alpha, *b2 = b, *v2 = v, *w2 = w;
    if (T > 0 && dk < d) {
      q2 = widen(q, rp.q, dk, E, 0);
      k2 = widen(k, rp.k, dk, E, 0);
      if (!(flags & GDN2_FLAG_SCALAR_ALPHA))  // layer prep: float32 log-decay, 0 = no decay
        al2 = (flags & GDN2_FLAG_LAYER_PREP) ? widen(alpha, rp.al, dk, 4, 0) : widen(alpha, rp.al, dk, E, one_bits);
      if (!(flags & GDN2_FLAG_SCALAR_B))
        b2 = widen(b, rp.b, dk, E, 0);
    }
    if (T > 0 && dv < d) {
      v2 = widen(v, rp.v, dv, E, 0);
      if (!(flags & GDN2_FLAG_SCALAR_W))
        w2 = widen(w, rp.w, dv, E, 0);
    }
    float *st2 = reinterpret_cast<float *>(wsr + rp.state);
    if (S0 && e == hipSuccess)
      e = gdn2::launch_pad(S0, st2, static_cast<long long>(N) * H, dk, dv, d, d, 4, 0, st);
    if (e != hipSuccess)
      return fail(GDN2_ERR_HIP, "gdn2_chunk_fwd: launch failed: %s", hipGetErrorString(e));
    void *o2 = dv < d ? static_cast<void *>(wsr + rp.o) : o;
    const gdn2_status_t s = gdn2_chunk_fwd(q2, k2, v2, al2, b2, w2, S0 ? st2 : nullptr, cu_seqlens, B, T, H, d, d,
                                           num_seqs, chunk, dt, flags, T > 0 ? o2 : o,
                                           S_final ? st2 : nullptr, wsr + rp.total, workspace_bytes - rp.total,
                                           stream);
    if (s != GDN2_OK)
      return s;  // the widened call's message stands
    if (T > 0 && dv < d)
      e = gdn2::launch_pad(o2, o, rows, 1, d, 1, dv, E, 0, st);
    if (S_final && e == hipSuccess)
      e = gdn2::launch_pad(st2, S_final, static_cast<long long>(N) * H, d, d, dk, dv, 4, 0, st);
    if (e != hipSuccess)
      return fail(GDN2_ERR_HIP, "gdn2_chunk_fwd: launch failed: %s", hipGetErrorString(e));
    return ok();
  }

  const size_t blk_bytes = r1_chunked ? r1_block_bytes_rt(dt, dk, chunk) : chunk_block_bytes_rt(dt, dk, chunk);
  if (blk_bytes == 0)
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_fwd: rule R1 on the chunked path needs bfloat16 or chunk 16 with dk = 128");
  const size_t need_exact = [&] {
    const size_t table = packed ? align256(static_cast<size_t>(N + 1) * sizeof(int32_t)) : 0;
    return table + static_cast<size_t>(num_slots_for(B, T, N, chunk, packed)) * H * blk_bytes;
  }();
  if (workspace_bytes < need_exact || (need_exact > 0 && !workspace))
    return fail(GDN2_ERR_WORKSPACE_TOO_SMALL,
                "gdn2_chunk_fwd: workspace of %zu bytes is smaller than the %zu needed",
                workspace_bytes, need_exact);
  // kept states go where the backward keeps its states (after the table and
  // the blocks, which sit where the forward puts them)
  const bwd_plan kp = keep ? plan_bwd(dt, B, T, H, dk, N, chunk, packed) : bwd_plan{};
  if (keep && (workspace_bytes < kp.table + kp.blocks + kp.states || !workspace))
    return fail(GDN2_ERR_WORKSPACE_TOO_SMALL,
                "gdn2_chunk_fwd: workspace of %zu bytes is smaller than the %zu needed to keep the states",
                workspace_bytes, kp.table + kp.blocks + kp.states);

  gdn2::chunk_args a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.al = alpha;
  a.b = b;
  a.w = w;
  a.S0 = S0;
  a.cu = cu_seqlens;
  a.B = B;
  a.T = T;
  a.H = H;
  a.num_seqs = N;
  a.num_slots = static_cast<int>(num_slots_for(B, T, N, chunk, packed));
  a.o = o;
  a.S_final = S_final;
  a.blk_bytes = blk_bytes;
  a.gates = ((flags & GDN2_FLAG_SCALAR_B) ? gdn2::GATE_SCALAR_B : 0u) |
            ((flags & GDN2_FLAG_SCALAR_W) ? gdn2::GATE_SCALAR_W : 0u) |
            ((flags & GDN2_FLAG_SCALAR_ALPHA) ? gdn2::GATE_SCALAR_ALPHA : 0u) |
            ((flags & GDN2_FLAG_LAYER_PREP) ? gdn2::GATE_LAYER_PREP : 0u);
  char *ws = static_cast<char *>(workspace);
  if (packed) {
    a.offsets = reinterpret_cast<int32_t *>(ws);
    a.blocks = ws + align256(static_cast<size_t>(N + 1) * sizeof(int32_t));
  } else {
    a.offsets = nullptr;
    a.blocks = ws;
  }
  if (keep)
    a.states = ws + kp.table + kp.blocks;
  if (T == 0) {
    // no tokens: the scan kernel alone copies S0 (or zeros) to S_final
    a.num_slots = 0;
  }
  if ((flags & GDN2_FLAG_FUSED) && !fused_available(dt, dk, chunk))
    return fail(GDN2_ERR_UNSUPPORTED, "gdn2_chunk_fwd: no single-pass kernel for dtype %d, dk=%d, chunk=%d",
                static_cast<int>(dt), dk, chunk);
  if (r1_chunked) {
    const hipError_t e = dispatch_chunk_r1(dt, dk, chunk, a, st);
    if (e != hipSuccess)
      return fail(GDN2_ERR_HIP, "gdn2_chunk_fwd: launch failed: %s", hipGetErrorString(e));
    return ok();
  }
  const seg_shape sx = seg_shape_of(B, T, N, chunk, packed);
  if ((flags & (path_flags | GDN2_FLAG_PREPARED)) == 0 && use_segments(sx, H) &&
      workspace_bytes >= plan_segments(dt, sx, H, dk, chunk).total) {
    const hipError_t e = run_segments(dt, dk, chunk, a, sx, ws, st);
    if (e != hipSuccess)
      return fail(GDN2_ERR_HIP, "gdn2_chunk_fwd: launch failed: %s", hipGetErrorString(e));
    return ok();
  }
  const hipError_t e = dispatch_chunk(dt, dk, chunk, a, flags, st);
  if (e != hipSuccess)
    return fail(GDN2_ERR_HIP, "gdn2_chunk_fwd: launch failed: %s", hipGetErrorString(e));
  return ok();
}

size_t gdn2_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int num_seqs, int chunk,
                                      gdn2_dtype_t dt) {
  if (B <= 0 || T < 0 || H <= 0 || !supported_dim(dk) || !supported_dim(dv) || !supported_chunk(chunk))
    return 0;
  if (dk != dv) {
    const int d = dk > dv ? dk : dv;
    const size_t inner = gdn2_chunk_bwd_workspace_bytes(B, T, H, d, d, num_seqs, chunk, dt);
    return inner == 0 ? 0 : plan_rect_bwd(B, T, H, dk, dv, num_seqs > 0 ? num_seqs : B).total + inner;
  }
  if (dt != GDN2_F32 && dt != GDN2_BF16)
    return 0;
  if (!sizes_supported(B, T, H, dk, B, chunk, false) ||
      (num_seqs > 0 && !sizes_supported(B, T, H, dk, num_seqs, chunk, true)))
    return 0;
  const int n = num_seqs > 0 ? num_seqs : B;
  const bwd_plan pf = plan_bwd(dt, B, T, H, dk, B, chunk, false);
  const bwd_plan pp = plan_bwd(dt, B, T, H, dk, n, chunk, true);
  const size_t plain = pf.total > pp.total ? pf.total : pp.total;
  // a few long sequences also take the segment schedule
  const seg_shape x = seg_shape_of(B, T, num_seqs, chunk, num_seqs > 0);
  return use_segments(x, H) ? align256(plain) + seg_bwd_extra(x, H, dk) : plain;
}

gdn2_status_t gdn2_chunk_bwd(const void *q, const void *k, const void *v, const void *alpha,
                             const void *b, const void *w, const float *S0,
                             const int32_t *cu_seqlens, int B, int T, int H, int dk, int dv,
                             int num_seqs, int chunk, gdn2_dtype_t dt, uint32_t flags,
                             const void *dout, const float *dS_final, void *dq, void *dk_out,
                             void *dv_out, void *dalpha, void *db, void *dw, float *dS0,
                             void *workspace, size_t workspace_bytes, void *stream) {
  if (dt != GDN2_F32 && dt != GDN2_BF16)
    return fail(GDN2_ERR_UNSUPPORTED, "gdn2_chunk_bwd: unknown dtype %d", static_cast<int>(dt));
  const uint32_t gate_flags = GDN2_FLAG_SCALAR_B | GDN2_FLAG_SCALAR_W | GDN2_FLAG_SCALAR_ALPHA | GDN2_FLAG_LAYER_PREP;
  if (flags & ~(gate_flags | GDN2_FLAG_PREPARED | GDN2_FLAG_KEEP_STATES))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_bwd: flags 0x%x: only the gate layout, layer prep, prepared-workspace and kept-states "
                "flags apply to the backward",
                flags);
  if ((flags & GDN2_FLAG_KEEP_STATES) && !(flags & GDN2_FLAG_PREPARED))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_bwd: GDN2_FLAG_KEEP_STATES comes with GDN2_FLAG_PREPARED (the forward's blocks and "
                "states)");
  if ((flags & GDN2_FLAG_PREPARED) && dk != dv)
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_bwd: GDN2_FLAG_PREPARED needs dk == dv (the widened call lays its workspace out "
                "differently from the forward's)");
  if (B <= 0 || T < 0 || H <= 0)
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_bwd: bad sizes B=%d T=%d H=%d", B, T, H);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_bwd: unsupported head dims dk=%d dv=%d (need dk, dv in {16,32,64,128})", dk, dv);
  if (!supported_chunk(chunk))
    return fail(GDN2_ERR_UNSUPPORTED, "gdn2_chunk_bwd: unsupported chunk %d (need 16 or 64)", chunk);
  const bool packed = cu_seqlens != nullptr;
  int N;
  if (packed) {
    if (B != 1)
      return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_bwd: packed input needs B == 1 (got %d)", B);
    if (num_seqs <= 0)
      return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_bwd: packed input needs num_seqs > 0");
    N = num_seqs;
  } else {
    if (num_seqs != 0 && num_seqs != B)
      return fail(GDN2_ERR_INVALID_ARGUMENT,
                  "gdn2_chunk_bwd: num_seqs=%d must be 0 or B=%d without cu_seqlens", num_seqs, B);
    N = B;
  }
  if (T > 0 && (!q || !k || !v || !alpha || !b || !w || !dout || !dq || !dk_out || !dv_out || !dalpha ||
                !db || !dw))
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_bwd: null input or gradient pointer");
  const void *ptrs[] = {q, k, v, alpha, b, w, S0, dout, dS_final, dq, dk_out, dv_out, dalpha, db, dw, dS0,
                        workspace};
  for (const void *p : ptrs)
    if (p && !aligned16(p))
      return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_bwd: pointers must be 16-byte aligned");
  if (!sizes_supported(B, T, H, dk > dv ? dk : dv, N, chunk, packed))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_bwd: sizes beyond the library's limits (at most 2^40 input elements, 2^24 chunk-heads, "
                "2^21 sequence-heads)");
  if (dk != dv) {
    // the square backward on d = max(dk, dv) (see gdn2_chunk_fwd): the
    // narrower side's inputs, dout and the states widened in the front of
    // the workspace, its gradients and dL/dS0 narrowed back; gradients of
    // the widened channels are dropped (those channels never reach o)
    const rect_bwd_plan rp = plan_rect_bwd(B, T, H, dk, dv, N);
    const int d = rp.d;
    if (workspace_bytes < rp.total || !workspace)
      return fail(GDN2_ERR_WORKSPACE_TOO_SMALL,
                  "gdn2_chunk_bwd: workspace of %zu bytes is smaller than the %zu needed to widen dk=%d dv=%d to %d",
                  workspace_bytes, rp.total, dk, dv, d);
    hipStream_t st = static_cast<hipStream_t>(stream);
    char *wsr = static_cast<char *>(workspace);
    const long long rows = static_cast<long long>(B) * T * H;
    const long long units = static_cast<long long>(N) * H;
    const int E = dt == GDN2_BF16 ? 2 : 4;
    const bool lp = (flags & GDN2_FLAG_LAYER_PREP) != 0;
    const uint32_t one_bits = dt == GDN2_BF16 ? 0x3F80u : 0x3F800000u;
    const void *in[6] = {q, k, v, alpha, b, w};
    void *grad[6] = {dq, dk_out, dv_out, dalpha, db, dw};
    const int width[6] = {dk, dk, dv, dk, dk, dv};
    const bool scalar[6] = {false, false, false, (flags & GDN2_FLAG_SCALAR_ALPHA) != 0,
                            (flags & GDN2_FLAG_SCALAR_B) != 0, (flags & GDN2_FLAG_SCALAR_W) != 0};
    const int esz[6] = {E, E, E, lp ? 4 : E, E, E};                // alpha: float32 log-decay under layer prep
    const uint32_t fill[6] = {0, 0, 0, lp ? 0u : one_bits, 0, 0};  // no decay on widened channels
    const void *in2[6];
    void *grad2[6];
    hipError_t e = hipSuccess;
    for (int i = 0; i < 6; ++i) {
      in2[i] = in[i];
      grad2[i] = grad[i];
      if (width[i] < d && !scalar[i] && T > 0) {
        if (e == hipSuccess)
          e = gdn2::launch_pad(in[i], wsr + rp.in[i], rows, 1, width[i], 1, d, esz[i], fill[i], st);
        in2[i] = wsr + rp.in[i];
        grad2[i] = wsr + rp.grad[i];
      }
    }
    const void *dout2 = dout;
    if (dv < d && T > 0) {
      if (e == hipSuccess)
        e = gdn2::launch_pad(dout, wsr + rp.dout, rows, 1, dv, 1, d, E, 0, st);
      dout2 = wsr + rp.dout;
    }
    float *s0w = reinterpret_cast<float *>(wsr + rp.s0), *dsfw = reinterpret_cast<float *>(wsr + rp.dsf),
          *ds0w = reinterpret_cast<float *>(wsr + rp.ds0);
    if (S0 && e == hipSuccess)
      e = gdn2::launch_pad(S0, s0w, units, dk, dv, d, d, 4, 0, st);
    if (dS_final && e == hipSuccess)
      e = gdn2::launch_pad(dS_final, dsfw, units, dk, dv, d, d, 4, 0, st);
    if (e != hipSuccess)
      return fail(GDN2_ERR_HIP, "gdn2_chunk_bwd: launch failed: %s", hipGetErrorString(e));
    const gdn2_status_t s = gdn2_chunk_bwd(
        in2[0], in2[1], in2[2], in2[3], in2[4], in2[5], S0 ? s0w : nullptr, cu_seqlens, B, T, H, d, d, num_seqs,
        chunk, dt, flags, dout2, dS_final ? dsfw : nullptr, grad2[0], grad2[1], grad2[2], grad2[3], grad2[4],
        grad2[5], dS0 ? ds0w : nullptr, wsr + rp.total, workspace_bytes - rp.total, stream);
    if (s != GDN2_OK)
      return s;  // the widened call's message stands
    for (int i = 0; i < 6; ++i)
      if (grad2[i] != grad[i] && e == hipSuccess)
        e = gdn2::launch_pad(grad2[i], grad[i], rows, 1, d, 1, width[i], esz[i], 0, st);
    if (dS0 && e == hipSuccess)
      e = gdn2::launch_pad(ds0w, dS0, units, d, d, dk, dv, 4, 0, st);
    if (e != hipSuccess)
      return fail(GDN2_ERR_HIP, "gdn2_chunk_bwd: launch failed: %s", hipGetErrorString(e));
    return ok();
  }
  const bwd_plan plan = plan_bwd(dt, B, T, H, dk, N, chunk, packed);
  if (workspace_bytes < plan.total || !workspace)
    return fail(GDN2_ERR_WORKSPACE_TOO_SMALL,
                "gdn2_chunk_bwd: workspace of %zu bytes is smaller than the %zu needed", workspace_bytes,
                plan.total);

  gdn2::bwd_args ba{};
  gdn2::chunk_args &a = ba.f;
  a.q = q;
  a.k = k;
  a.v = v;
  a.al = alpha;
  a.b = b;
  a.w = w;
  a.S0 = S0;
  a.cu = cu_seqlens;
  a.B = B;
  a.T = T;
  a.H = H;
  a.num_seqs = N;
  a.num_slots = T == 0 ? 0 : static_cast<int>(num_slots_for(B, T, N, chunk, packed));
  a.o = nullptr;
  a.S_final = nullptr;
  a.blk_bytes = chunk_block_bytes_rt(dt, dk, chunk);
  a.gates = ((flags & GDN2_FLAG_SCALAR_B) ? gdn2::GATE_SCALAR_B : 0u) |
            ((flags & GDN2_FLAG_SCALAR_W) ? gdn2::GATE_SCALAR_W : 0u) |
            ((flags & GDN2_FLAG_SCALAR_ALPHA) ? gdn2::GATE_SCALAR_ALPHA : 0u) |
            ((flags & GDN2_FLAG_LAYER_PREP) ? gdn2::GATE_LAYER_PREP : 0u);
  char *ws = static_cast<char *>(workspace);
  a.offsets = packed ? reinterpret_cast<int32_t *>(ws) : nullptr;
  a.blocks = ws + plan.table;
  a.states = ws + plan.table + plan.blocks;
  ba.dstates = ws + plan.table + plan.blocks + plan.states;
  ba.pwflag = reinterpret_cast<unsigned char *>(ws + plan.table + plan.blocks + plan.states + plan.dstates);
  ba.dout = dout;
  ba.dSf = dS_final;
  ba.dS0 = dS0;
  ba.dq = dq;
  ba.dk = dk_out;
  ba.dv = dv_out;
  ba.dal = dalpha;
  ba.db = db;
  ba.dw = dw;
  // a few long sequences: the segment schedule, when the workspace holds it
  seg_run sr{};
  const seg_run *sgp = nullptr;
  const seg_shape sx = seg_shape_of(B, T, N, chunk, packed);
  if (use_segments(sx, H)) {
    size_t cb = 0;
    int G = 0;
    const size_t extra = seg_bwd_extra(sx, H, dk, &cb, &G);
    if (workspace_bytes >= align256(plan.total) + extra) {
      sr.ws = ws + align256(plan.total);
      sr.cu_bytes = cb;
      sr.N = sx.N;
      sr.G = G;
      sr.T_total = sx.T_total;
      sgp = &sr;
    }
  }
  const hipError_t e =
      dispatch_bwd(dt, dk, chunk, ba, sgp, (flags & GDN2_FLAG_PREPARED) != 0,
                   (flags & GDN2_FLAG_KEEP_STATES) != 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(GDN2_ERR_HIP, "gdn2_chunk_bwd: launch failed: %s", hipGetErrorString(e));
  return ok();
}

gdn2_status_t gdn2_chunk_segment_map(const void *q, const void *k, const void *v, const void *alpha,
                                     const void *b, const void *w, const int32_t *cu_seqlens, int B, int T,
                                     int H, int dk, int dv, int num_seqs, int chunk, gdn2_dtype_t dt,
                                     uint32_t flags, float *Phi, float *Psi, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  if (dt != GDN2_F32 && dt != GDN2_BF16)
    return fail(GDN2_ERR_UNSUPPORTED, "gdn2_chunk_segment_map: unknown dtype %d", static_cast<int>(dt));
  const uint32_t gate_flags = GDN2_FLAG_SCALAR_B | GDN2_FLAG_SCALAR_W | GDN2_FLAG_SCALAR_ALPHA | GDN2_FLAG_LAYER_PREP;
  if (flags & ~gate_flags)
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_segment_map: flags 0x%x: only the gate layout and layer prep flags apply", flags);
  if (B <= 0 || T < 0 || H <= 0)
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_segment_map: bad sizes B=%d T=%d H=%d", B, T, H);
  if (dk != dv || !supported_dim(dk))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_segment_map: unsupported head dims dk=%d dv=%d (need dk == dv in {16,32,64,128})",
                dk, dv);
  if (!supported_chunk(chunk))
    return fail(GDN2_ERR_UNSUPPORTED, "gdn2_chunk_segment_map: unsupported chunk %d (need 16 or 64)", chunk);
  const bool packed = cu_seqlens != nullptr;
  int N;
  if (packed) {
    if (B != 1)
      return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_segment_map: packed input needs B == 1 (got %d)", B);
    if (num_seqs <= 0)
      return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_segment_map: packed input needs num_seqs > 0");
    N = num_seqs;
  } else {
    if (num_seqs != 0 && num_seqs != B)
      return fail(GDN2_ERR_INVALID_ARGUMENT,
                  "gdn2_chunk_segment_map: num_seqs=%d must be 0 or B=%d without cu_seqlens", num_seqs, B);
    N = B;
  }
  if (!Phi || !Psi)
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_segment_map: null Phi or Psi");
  if (T > 0 && (!q || !k || !v || !alpha || !b || !w))
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_segment_map: null input pointer");
  const void *ptrs[] = {q, k, v, alpha, b, w, Phi, Psi, workspace};
  for (const void *p : ptrs)
    if (p && !aligned16(p))
      return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_segment_map: pointers must be 16-byte aligned");
  if (!sizes_supported(B, T, H, dk, N, chunk, packed))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_segment_map: sizes beyond the library's limits (at most 2^40 input elements, 2^24 chunk-heads, "
                "2^21 sequence-heads)");
  const size_t table = packed ? align256(static_cast<size_t>(N + 1) * sizeof(int32_t)) : 0;
  const size_t need = table + static_cast<size_t>(num_slots_for(B, T, N, chunk, packed)) * H *
                                  chunk_block_bytes_rt(dt, dk, chunk);
  if (workspace_bytes < need || !workspace)
    return fail(GDN2_ERR_WORKSPACE_TOO_SMALL,
                "gdn2_chunk_segment_map: workspace of %zu bytes is smaller than the %zu needed",
                workspace_bytes, need);
  gdn2::chunk_args a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.al = alpha;
  a.b = b;
  a.w = w;
  a.cu = cu_seqlens;
  a.B = B;
  a.T = T;
  a.H = H;
  a.num_seqs = N;
  a.num_slots = T == 0 ? 0 : static_cast<int>(num_slots_for(B, T, N, chunk, packed));
  a.blk_bytes = chunk_block_bytes_rt(dt, dk, chunk);
  a.gates = ((flags & GDN2_FLAG_SCALAR_B) ? gdn2::GATE_SCALAR_B : 0u) |
            ((flags & GDN2_FLAG_SCALAR_W) ? gdn2::GATE_SCALAR_W : 0u) |
            ((flags & GDN2_FLAG_SCALAR_ALPHA) ? gdn2::GATE_SCALAR_ALPHA : 0u) |
            ((flags & GDN2_FLAG_LAYER_PREP) ? gdn2::GATE_LAYER_PREP : 0u);
  char *ws = static_cast<char *>(workspace);
  a.offsets = packed ? reinterpret_cast<int32_t *>(ws) : nullptr;
  a.blocks = ws + table;
  const hipError_t e = dispatch_segmap(dt, dk, chunk, a, Phi, Psi, static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(GDN2_ERR_HIP, "gdn2_chunk_segment_map: launch failed: %s", hipGetErrorString(e));
  return ok();
}

gdn2_status_t gdn2_segment_combine(const float *Phi, const float *Psi, const float *S0, int G, int H, int dk,
                                   int dv, float *S_in, float *S_final, void *stream) {
  if (G < 0 || H <= 0)
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_segment_combine: bad sizes G=%d H=%d", G, H);
  if (dk != dv || !supported_dim(dk))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_segment_combine: unsupported head dims dk=%d dv=%d (need dk == dv in {16,32,64,128})",
                dk, dv);
  if (G > 0 && (!Phi || !Psi || !S_in))
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_segment_combine: null Phi, Psi or S_in");
  const void *ptrs[] = {Phi, Psi, S0, S_in, S_final};
  for (const void *p : ptrs)
    if (p && !aligned16(p))
      return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_segment_combine: pointers must be 16-byte aligned");
  if (G == 0 && !S_final)
    return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipErrorInvalidValue;
  {
    prof_scope p("segment_combine", st);
    switch (dk) {
      case 16: e = gdn2::launch_seg_combine<16>(Phi, Psi, S0, G, H, 1, S_in, S_final, st); break;
      case 32: e = gdn2::launch_seg_combine<32>(Phi, Psi, S0, G, H, 1, S_in, S_final, st); break;
      case 64: e = gdn2::launch_seg_combine<64>(Phi, Psi, S0, G, H, 1, S_in, S_final, st); break;
      case 128: e = gdn2::launch_seg_combine<128>(Phi, Psi, S0, G, H, 1, S_in, S_final, st); break;
    }
  }
  if (e != hipSuccess)
    return fail(GDN2_ERR_HIP, "gdn2_segment_combine: launch failed: %s", hipGetErrorString(e));
  return ok();
}

gdn2_status_t gdn2_decode_step(const void *q, const void *k, const void *v, const void *alpha,
                               const void *b, const void *w, float *S, void *o, int N, int H,
                               int dk, int dv, gdn2_dtype_t dt, void *stream) {
  if (dt != GDN2_F32 && dt != GDN2_BF16)
    return fail(GDN2_ERR_UNSUPPORTED, "gdn2_decode_step: unknown dtype %d", static_cast<int>(dt));
  if (N <= 0 || H <= 0)
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_decode_step: bad sizes N=%d H=%d", N, H);
  if (!supported_dim(dk) || !supported_dim(dv))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_decode_step: unsupported head dims dk=%d dv=%d (need dk, dv in {16,32,64,128})", dk, dv);
  if (!q || !k || !v || !alpha || !b || !w || !S || !o)
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_decode_step: null pointer");
  const void *ptrs[] = {q, k, v, alpha, b, w, S, o};
  for (const void *p : ptrs)
    if (!aligned16(p))
      return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_decode_step: pointers must be 16-byte aligned");
  if (static_cast<long long>(N) * H > (1LL << 24) - 1)  // one workgroup of 256 threads per sequence-head
    return fail(GDN2_ERR_UNSUPPORTED, "gdn2_decode_step: too many sequence-heads (at most 2^24 - 1)");
  const hipError_t e = dispatch_decode(dt, dk, dv, q, k, v, alpha, b, w, S, o, N, H,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess)
    return fail(GDN2_ERR_HIP, "gdn2_decode_step: launch failed: %s", hipGetErrorString(e));
  return ok();
}

gdn2_status_t gdn2_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *alpha,
                                     const void *b, const void *w, const float *S0,
                                     const int32_t *cu_seqlens, int B, int T, int H, int dk, int dv,
                                     int num_seqs, int chunk, gdn2_dtype_t dt, uint32_t flags, void *o,
                                     float *S_final, void *stream) {
  const uint32_t gate_flags = GDN2_FLAG_SCALAR_B | GDN2_FLAG_SCALAR_W | GDN2_FLAG_SCALAR_ALPHA | GDN2_FLAG_LAYER_PREP;
  if (flags & ~(gate_flags | GDN2_FLAG_TWO_PASS))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_fwd_noalloc: flags 0x%x: only the gate layout and layer prep flags apply "
                "(it runs the two-pass kernels)", flags);
  if (dt != GDN2_F32 && dt != GDN2_BF16)
    return fail(GDN2_ERR_UNSUPPORTED, "gdn2_chunk_fwd_noalloc: unknown dtype %d", static_cast<int>(dt));
  if (B <= 0 || T < 0 || H <= 0)
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_fwd_noalloc: bad sizes B=%d T=%d H=%d", B, T, H);
  if (dk != dv || !supported_dim(dk) || !supported_chunk(chunk))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_fwd_noalloc: unsupported dk=%d dv=%d chunk=%d (need dk == dv in {16,32,64,128}, "
                "chunk 16 or 64)", dk, dv, chunk);
  if (T > 0 && (!q || !k || !v || !alpha || !b || !w || !o))
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_fwd_noalloc: null input or output pointer");
  flags |= GDN2_FLAG_TWO_PASS;
  const size_t cap = GDN2_NOALLOC_SCRATCH_BYTES;
  const bool packed = cu_seqlens != nullptr;
  if (packed && num_seqs <= 0)
    return fail(GDN2_ERR_INVALID_ARGUMENT, "gdn2_chunk_fwd_noalloc: packed input needs num_seqs > 0");
  if (!sizes_supported(B, T, H, dk, packed ? num_seqs : B, chunk, packed))
    return fail(GDN2_ERR_UNSUPPORTED,
                "gdn2_chunk_fwd_noalloc: sizes beyond the library's limits (at most 2^40 input elements, "
                "2^24 chunk-heads, 2^21 sequence-heads)");
  // the plain two-pass workspace of the whole call, as gdn2_chunk_fwd checks it
  const size_t whole_plain = (packed ? align256(static_cast<size_t>(num_seqs + 1) * sizeof(int32_t)) : 0) +
                             static_cast<size_t>(num_slots_for(B, T, packed ? num_seqs : B, chunk, packed)) * H *
                                 chunk_block_bytes_rt(dt, dk, chunk);
  if (packed && whole_plain > cap)
    return fail(GDN2_ERR_WORKSPACE_TOO_SMALL,
                "gdn2_chunk_fwd_noalloc: packed input needs %zu bytes of scratch, more than the %zu the "
                "library holds; split the call", whole_plain, cap);
  hipError_t herr = hipSuccess;
  if (whole_plain <= cap) {
    char *ws = static_cast<char *>(device_scratch(&herr));
    if (!ws)
      return fail(GDN2_ERR_HIP, "gdn2_chunk_fwd_noalloc: scratch address: %s", hipGetErrorString(herr));
    return gdn2_chunk_fwd(q, k, v, alpha, b, w, S0, cu_seqlens, B, T, H, dk, dv, num_seqs, chunk, dt, flags, o,
                          S_final, ws, cap, stream);
  }
  // Fixed-length input too large for the scratch in one call: every
  // sequence in pieces of whole chunks, run in order, each from the state
  // the previous piece left (in S_final, or in the scratch's first bytes).
  // Pieces of whole chunks reproduce the single call's results exactly.
  if (num_seqs != 0 && num_seqs != B)
    return fail(GDN2_ERR_INVALID_ARGUMENT,
                "gdn2_chunk_fwd_noalloc: num_seqs=%d must be 0 or B=%d without cu_seqlens", num_seqs, B);
  const size_t carry = S_final ? 0 : align256(static_cast<size_t>(H) * dk * dv * sizeof(float));
  const size_t per_chunk = static_cast<size_t>(H) * chunk_block_bytes_rt(dt, dk, chunk);
  const long max_chunks = cap > carry ? static_cast<long>((cap - carry) / per_chunk) : 0;
  if (max_chunks < 1)
    return fail(GDN2_ERR_WORKSPACE_TOO_SMALL,
                "gdn2_chunk_fwd_noalloc: one chunk of %d heads needs %zu bytes of scratch, more than the %zu "
                "the library holds", H, per_chunk + carry, cap);
  const int Tp = static_cast<int>(max_chunks > T / chunk + 1 ? T / chunk + 1 : max_chunks) * chunk;
  const size_t el = dt == GDN2_BF16 ? 2 : 4;
  // bytes per token of each tensor: [.., H, width] rows of its element type
  const size_t row_q = static_cast<size_t>(H) * dk * el, row_v = static_cast<size_t>(H) * dv * el;
  const size_t row_a = static_cast<size_t>(H) * ((flags & GDN2_FLAG_SCALAR_ALPHA) ? 1 : dk) *
                       ((flags & GDN2_FLAG_LAYER_PREP) ? 4 : el);
  const size_t row_b = static_cast<size_t>(H) * ((flags & GDN2_FLAG_SCALAR_B) ? 1 : dk) * el;
  const size_t row_w = static_cast<size_t>(H) * ((flags & GDN2_FLAG_SCALAR_W) ? 1 : dv) * el;
  const size_t st = static_cast<size_t>(H) * dk * dv;  // floats per sequence state
  char *ws = static_cast<char *>(device_scratch(&herr));
  if (!ws)
    return fail(GDN2_ERR_HIP, "gdn2_chunk_fwd_noalloc: scratch address: %s", hipGetErrorString(herr));
  float *carry_p = reinterpret_cast<float *>(ws);
  for (int n = 0; n < B; ++n) {
    for (int t0 = 0; t0 < T; t0 += Tp) {
      const int len = T - t0 < Tp ? T - t0 : Tp;
      const size_t tok = static_cast<size_t>(n) * T + t0;
      auto at = [&](const void *p, size_t row) {
        return p ? static_cast<const void *>(static_cast<const char *>(p) + tok * row) : nullptr;
      };
      const void *pa = at(alpha, row_a), *pb = at(b, row_b), *pw = at(w, row_w);
      for (const void *p : {pa, pb, pw})
        if (p && !aligned16(p))
          return fail(GDN2_ERR_UNSUPPORTED,
                      "gdn2_chunk_fwd_noalloc: the call needs %zu bytes of scratch (more than %zu) and its "
                      "pieces of %d tokens would leave a per-(token, head) gate 16-byte misaligned",
                      whole_plain, cap, Tp);
      const float *s_in = t0 == 0 ? (S0 ? S0 + n * st : nullptr) : (S_final ? S_final + n * st : carry_p);
      float *s_out = S_final ? S_final + n * st : (t0 + len < T ? carry_p : nullptr);
      const gdn2_status_t r = gdn2_chunk_fwd(
          at(q, row_q), at(k, row_q), at(v, row_v), pa, pb, pw, s_in, nullptr, 1, len, H, dk, dv, 0, chunk, dt,
          flags, static_cast<char *>(o) + tok * row_v, s_out, ws + carry, cap - carry, stream);
      if (r != GDN2_OK)
        return r;
    }
  }
  return ok();
}

const char *gdn2_status_string(gdn2_status_t status) {
  switch (status) {
  case GDN2_OK:
    return "ok";
  case GDN2_ERR_INVALID_ARGUMENT:
    return "invalid argument";
  case GDN2_ERR_UNSUPPORTED:
    return "unsupported";
  case GDN2_ERR_WORKSPACE_TOO_SMALL:
    return "workspace too small";
  case GDN2_ERR_HIP:
    return "HIP error";
  default:
    break;
  }
  return "unknown status";
}

const char *gdn2_last_error(void) { return g_last_error.c_str(); }

int gdn2_abi_version(void) { return GDN2_ABI_VERSION; }

gdn2_status_t gdn2_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = on != 0;
  return ok();
}

gdn2_status_t gdn2_profile_read(int max_kernels, const char **names, double *total_ms, int *counts,
                                int *n_kernels, int reset) {
  std::vector<prof_rec> pend;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    pend.swap(g_prof_pending);
  }
  for (prof_rec &r : pend) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e == hipSuccess)
      e = hipEventElapsedTime(&ms, r.start, r.stop);
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
    if (e != hipSuccess)
      return fail(GDN2_ERR_HIP, "gdn2_profile_read: %s", hipGetErrorString(e));
    std::lock_guard<std::mutex> lk(g_prof_mu);
    bool found = false;
    for (auto &kv : g_prof_total) {
      if (kv.first == r.name) {
        kv.second.first += ms;
        kv.second.second += 1;
        found = true;
        break;
      }
    }
    if (!found)
      g_prof_total.push_back({r.name, {static_cast<double>(ms), 1}});
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int n = 0;
  for (auto &kv : g_prof_total) {
    if (n < max_kernels) {
      if (names)
        names[n] = kv.first;
      if (total_ms)
        total_ms[n] = kv.second.first;
      if (counts)
        counts[n] = kv.second.second;
    }
    ++n;
  }
  if (n_kernels)
    *n_kernels = n;
  if (reset)
    g_prof_total.clear();
  return ok();
}

}  // extern "C"
