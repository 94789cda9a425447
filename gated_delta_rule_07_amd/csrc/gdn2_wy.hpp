// gdn2_wy.hpp -- the per-chunk part of the chunkwise GDN-2 forward, shared by
// the two-pass path (gdn2_chunk.hip) and the fused path (gdn2_fused.hip).
//
// The recurrence (gdn2_recurrent.hip) is re-parallelised over chunks of C
// tokens, as the pages describe: split the sequence into chunks, use matrix
// products inside each chunk, build in-chunk WY auxiliary matrices with the
// erase gate inside the key products and the write gate inside the delta
// values, and absorb the per-channel decay into the erase factors (aixai.ru
// blog, implementation section; aiexpert.news/pt, method paragraph).
//
// Derivation used here (one head, one chunk, tokens t = 1..C, entering state
// S0).  With g_t the running sum of log alpha from the chunk start and
// gamma_t = exp(g_t) (per key channel), write S_t = Diag(gamma_t) X_t.  Then
// X_t = X_{t-1} + khat_t z_t^T with khat_t = k_t / gamma_t, and
//   z_t = w_t (.) v_t - X_{t-1}^T echk_t,   echk_t = b_t (.) k_t (.) gamma_t.
// Collecting the C delta values z_t in Z (C x dv):
//   (I + A) Z = U - E S0,  A = strict_lower(E Khat^T),  U_t = w_t (.) v_t
//   Z = Ut - W S0          with T = (I + A)^{-1}, W = T E, Ut = T U
//   O = Qchk S0 + P Z      with Qchk_t = q_t (.) gamma_t, P = lower_incl(Qchk Khat^T)
//     = Q' S0 + O_intra    with Q' = Qchk - P W, O_intra = P Ut
//   S_C = Diag(gamma_C) S0 + Kbar^T Z,   Kbar_t = k_t (.) gamma_C / gamma_t.
// W, Ut, Q', O_intra, Kbar and gamma_C depend only on the chunk's own inputs;
// the entering state only enters through three state-sized products.
//
// Numerics of the decay factorisation: every factor exp(g_t - g_s) with s <= t
// is at most 1, but splitting it as gamma_t / gamma_s can overflow, and with
// alpha = 0 (log -inf) a difference of two prefix sums is -inf - (-inf).
// Every factor below is therefore a sum of log decays taken directly (a
// prefix or suffix scan, or a sum of whole sub-blocks), never a difference,
// and is at most 1, except on the diagonal blocks.  Per 16-token sub-block
// I (rho_I = g just before it):
//   rows     e^{g_t - rho_I}  (prefix within the sub-block)
//   keys     e^{rho_{I+1} - g_s} (suffix within the sub-block: the key
//            referenced to the END of its own sub-block)
//   between  e^{rho_I - rho_{J+1}} (whole sub-blocks J+1 .. I-1), folded into
//            the keys of sub-block J for row sub-block I > J
//   A[t][s] = sum_c (b k_t e^{g_t - rho_I}) (k_s e^{rho_{J+1} - g_s}) e^{rho_I - rho_{J+1}}
// E, Qchk use the chunk start (e^{g_t} = e^{rho_I} e^{g_t - rho_I}) and Kbar
// the chunk end (e^{g_C - g_s} = e^{rho_{J+1} - g_s} e^{g_C - rho_{J+1}}).
// The diagonal blocks (s, t in one sub-block) take the key factor
// e^{rho_I - g_s} <= e^{-(sub-block's log decay)}: while every channel's
// decay over the sub-block is above 2^-64 that is bounded and the block is
// one matrix-core product; otherwise (very strong decay, alpha = 0) the
// sub-block's wave forms the block pairwise, token by token, with running
// products of the alphas themselves (wy_diag_pairwise).

// Work split inside a workgroup of C/16 waves (the "wy" phases below):
//   rows     wave I owns the 16-token sub-block I: loads of q, k, alpha, b,
//            log2(alpha) and its prefix sum over tokens (DPP row scan), the
//            decayed/gated operands, the A and P rows of sub-block I, and the
//            rows of T = (I + A)^{-1} (16x16 diagonal inverse by forward
//            substitution, one column per lane; off-diagonal blocks level by
//            level with T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ on matrix cores)
//   columns  wave I owns a range of 16-wide column tiles of dk (W, Q') and of
//            dv (Ut, O_intra), so the matrix work of phases 4-5 is balanced.
// Matrix products use the fragment convention of gdn2_device.hpp; results are
// produced directly in the layout their consumer reads.
#pragma once

#include "gdn2_device.hpp"
#include "gdn2_kernels.hpp"

namespace gdn2 {

// raw 4-element loads (kept packed until first use)
template <typename IO> struct raw4;
template <> struct raw4<float> {
  f32x4 x;
  __device__ static __forceinline__ raw4 ld(const float *p) {
    raw4 r;
    r.x = *reinterpret_cast<const f32x4 *>(p);
    return r;
  }
  __device__ static __forceinline__ raw4 fill(float v) {
    raw4 r;
    r.x = f32x4{v, v, v, v};
    return r;
  }
  __device__ static __forceinline__ raw4 splat(float e) { return fill(e); }
  // one element parked in slot 0 (the others unspecified) and read back
  __device__ static __forceinline__ raw4 first(float e) {
    raw4 r;
    r.x[0] = e;
    return r;
  }
  __device__ __forceinline__ float first() const { return x[0]; }
  // x where keep, else four copies of e
  __device__ static __forceinline__ raw4 select(bool keep, const raw4 &x, float e) {
    return keep ? x : fill(e);
  }
  __device__ __forceinline__ f32x4 f() const { return x; }
};
template <> struct raw4<bf16_t> {
  uint2 x;
  __device__ static __forceinline__ raw4 ld(const bf16_t *p) {
    raw4 r;
    r.x = *reinterpret_cast<const uint2 *>(p);
    return r;
  }
  __device__ static __forceinline__ raw4 fill(float v) { return splat(f2bf(v)); }
  // four copies of one stored element
  __device__ static __forceinline__ raw4 splat(bf16_t e) {
    raw4 r;
    r.x.x = static_cast<uint32_t>(e) | (static_cast<uint32_t>(e) << 16);
    r.x.y = r.x.x;
    return r;
  }
  __device__ static __forceinline__ raw4 first(bf16_t e) {
    raw4 r;
    r.x.x = e;
    return r;
  }
  __device__ __forceinline__ bf16_t first() const { return static_cast<bf16_t>(x.x & 0xffffu); }
  __device__ static __forceinline__ raw4 select(bool keep, const raw4 &x, float e) {
    const raw4 f = fill(e);
    raw4 r;
    r.x.x = keep ? x.x.x : f.x.x;
    r.x.y = keep ? x.x.y : f.x.y;
    return r;
  }
  __device__ __forceinline__ f32x4 f() const {
    f32x4 r;
    r[0] = __builtin_bit_cast(float, x.x << 16);
    r[1] = __builtin_bit_cast(float, x.x & 0xffff0000u);
    r[2] = __builtin_bit_cast(float, x.y << 16);
    r[3] = __builtin_bit_cast(float, x.y & 0xffff0000u);
    return r;
  }
};

__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Per (chunk, head) block of intermediates, all tiles fragment-ordered.  The
// first SHARED bytes (-W, Q', Kbar^T, gamma_C and the lower-triangular tiles
// of P) are what every column slice of the state scan needs; the scan copies
// them to LDS as one block and forms O_intra = P Ut itself from P and the Ut
// tiles it reads anyway (P's tiles are a third of O_intra's bytes, so the
// block is 13 % smaller for bf16, d = 128, C = 64).  A operands of the scan
// are stored with their 16-wide k tiles paired (tile_off), so one 16-byte
// load yields a 16x16x32 operand.  The fused kernel keeps the first SHARED0
// bytes in LDS.
template <typename IO, int D, int C> struct blk_layout {
  static constexpr int NB = C / 16, NK = D / 16, NT = NB * (NB + 1) / 2;
  static constexpr size_t TB = frag<IO>::TILE_BYTES;
  static constexpr size_t WN = 0;                   // rows tt, k tiles over dk: RowFrag(-W)
  static constexpr size_t QP = WN + NB * NK * TB;   // rows tt, k tiles over dk: RowFrag(Q')
  static constexpr size_t KB = QP + NB * NK * TB;   // rows dk tile, k tiles over tokens: RowFrag(Kbar^T)
  static constexpr size_t GAM = KB + NK * NB * TB;  // [D] float gamma_C
  static constexpr size_t SHARED0 = (GAM + D * sizeof(float) + 1023) & ~static_cast<size_t>(1023);
  static constexpr size_t P = SHARED0;              // NT tiles RowFrag(P_IJ), J <= I, at tri_index(I, J)
  static constexpr size_t SHARED = (P + NT * TB + 1023) & ~static_cast<size_t>(1023);
  static constexpr size_t UT = SHARED;              // rows tt, dv tiles paired: ColFrag(Ut)
  static constexpr size_t BYTES = align256(UT + NB * NK * TB);
};

// The block of rule R1 (gdn2_rule_r1.hip): the default block's -W', Q'',
// Ebar^T and gamma_C slots (its first SHARED0 bytes), then -Ut' (ColFrag),
// O'' (RowFrag) and N = Kbar^T U (ColFrag tiles, dk tile x dv tile).
template <typename IO, int D, int C> struct r1_layout {
  typedef blk_layout<IO, D, C> L;
  static constexpr int NB = C / 16, NK = D / 16;
  static constexpr size_t TB = L::TB;
  static constexpr size_t UT = L::SHARED0;            // rows tt, dv tiles paired: ColFrag(-Ut')
  static constexpr size_t OI = UT + NB * NK * TB;     // rows tt, dv tiles paired: RowFrag(O'')
  static constexpr size_t NC = OI + NB * NK * TB;     // dk tiles x dv tiles: ColFrag(N)
  static constexpr size_t BYTES = align256(NC + NK * NK * TB);
};

// chunk slot -> (sequence, first token (flat index), valid length)
template <int C>
__device__ __forceinline__ bool locate_chunk(int slot, const chunk_args &a, int &seq, long &t0,
                                             int &len) {
  if (a.cu) {
    const int total = a.offsets[a.num_seqs];
    if (slot >= total)
      return false;
    int lo = 0, hi = a.num_seqs - 1;  // largest n with offsets[n] <= slot
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (a.offsets[mid] <= slot)
        lo = mid;
      else
        hi = mid - 1;
    }
    seq = lo;
    t0 = static_cast<long>(a.cu[lo]) + static_cast<long>(slot - a.offsets[lo]) * C;
    const long rem = static_cast<long>(a.cu[lo + 1]) - t0;
    len = rem < C ? static_cast<int>(rem) : C;
    return true;
  }
  const int nc = (a.T + C - 1) / C;
  seq = slot / nc;
  const int c = slot - seq * nc;
  t0 = static_cast<long>(seq) * a.T + static_cast<long>(c) * C;
  len = (a.T - c * C) < C ? (a.T - c * C) : C;
  return seq < a.num_seqs;
}

// sequence n -> (first chunk slot, chunk count, first token, end token)
template <int C>
__device__ __forceinline__ void sequence_range(int n, const chunk_args &a, int &c_begin, int &nchunks,
                                               long &tstart, long &tend) {
  if (a.cu) {
    c_begin = a.offsets[n];
    nchunks = a.offsets[n + 1] - c_begin;
    tstart = a.cu[n];
    tend = a.cu[n + 1];
  } else {
    const int nc = (a.T + C - 1) / C;
    c_begin = n * nc;
    nchunks = nc;
    tstart = static_cast<long>(n) * a.T;
    tend = tstart + a.T;
  }
}

template <typename IO, int D, int C> struct wy_smem {
  static constexpr int NB = C / 16, NK = D / 16;
  static constexpr int NP = NB * (NB - 1) / 2;  // sub-block pairs J < I
  static constexpr int NT = NB * (NB + 1) / 2;  // sub-block pairs J <= I
  static constexpr int NKS = (NP > NB ? NP : NB);
  static constexpr int TB = frag<IO>::TILE_BYTES;
  float tot[NB][D];                  // per-sub-block sum of log2(alpha)
  float f1[NB][D];                   // exp2(rho_I): decay from chunk start to sub-block I
  float f2[NB][D];                   // exp2(g_C - rho_{I+1}): decay after sub-block I to chunk end
  float sig[NP > 0 ? NP : 1][D];     // exp2(rho_I - rho_{J+1}) <= 1 for the pair (I, J), J < I
  float ad[NB][16][16];              // diagonal blocks of A, row-major
  // RowFrag(k_s e^{rho_I - g_s}) (keys of sub-block J for rows of sub-block
  // I, J < I) for each pair (I, J), k tiles paired; after the
  // A/P products the same bytes hold RowFrag(Qchk) tiles [NB][NK]
  alignas(16) unsigned char khs[NKS][NK][TB];
  alignas(16) unsigned char ec[NB][NK][TB];  // ColFrag(E_J), one tile per 16 channels
  alignas(16) unsigned char pr[NT][TB];      // RowFrag(P_IJ)
  alignas(16) unsigned char tcol[NT][TB];    // ColFrag(T_IJ)
  alignas(16) unsigned char trow[NT][TB];    // RowFrag(T_IJ)
};

__device__ __forceinline__ constexpr int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }
__device__ __forceinline__ constexpr int tri_index(int I, int J) { return I * (I + 1) / 2 + J; }

// Per-wave registers of one chunk's row phases.
// Rows of q, k, b, alpha held by one lane.  With layer prep (LP) alpha is
// kept as log2 of the decay in float32 (lg), and q, k are the raw rows.
template <typename IO, int D, bool LP = false> struct wy_rows {
  static constexpr int NK = D / 16;
  raw4<IO> q[NK], k[NK], b[NK];
  raw4<IO> al[LP ? 1 : NK];
  f32x4 lg[LP ? NK : 1];
};

__device__ __forceinline__ float fast_sigmoid(float x) {
  return __builtin_amdgcn_rcpf(1.f + fast_exp2(-1.4426950408889634f * x));
}

// Loads row t (of the chunk starting at token t0) of q, k, b, alpha: this
// lane's four channels 16kk + 4g .. +3 of every 16-channel tile.  Rows past
// the valid length read as zeros (alpha as one, i.e. no decay).  With
// GATE_SCALAR_B / GATE_SCALAR_ALPHA, b / alpha are one element per (token,
// head), repeated over the channels.
// Input modes of the loaders (compile-time): GM_PLAIN, every gate per
// channel; GM_KDA, b and w per (token, head); GM_GDN, b, w and alpha per
// (token, head); GM_GATES, any of them per (token, head), read from the
// GATE_SCALAR_* bits of chunk_args::gates at run time; GM_LAYER, layer prep
// (raw q, k, gate logits, float32 log decay) with the same run-time bits.
constexpr int GM_PLAIN = 0, GM_GATES = 1, GM_LAYER = 2, GM_KDA = 3, GM_GDN = 4;

// Loads the inputs of one chunk, with the gate layouts fixed at compile time
// (SB, SW, SA: b, w, alpha one element per (token, head)):
//  - rows of q, k, b, alpha for token t = 16 I + m of the lane (wy_rows);
//  - v and w of all C tokens for NVW column tiles starting at vt0 (RowFrag
//    layout: lane (m, g) holds row 16J + m, columns 16vt + 4g .. +3).
// Rows past the end must act as absent: k = 0, v = 0 and alpha = 1 (no
// decay).  Their loads read the chunk's first row instead (always in the
// sequence; element `row` exists in either gate layout), unconditionally, and
// the masks are applied only after every load has issued: no branch and no
// consumer sits between the loads, so no memory round trip is paid before
// the others start.  k = 0 and v = 0 remove b and w of those rows, and q only
// reaches their own (unstored) outputs, so b, w and q need no mask.  With
// layer prep (LP) alpha is the float32 natural-log decay, kept as log2 in lg.
template <typename IO, int D, int C, int NVW, bool LP, bool SB, bool SW, bool SA>
__device__ __forceinline__ void wy_load_chunk_t(const chunk_args &a, long t0, int len, int h, int I, int vt0,
                                                bool owner, int m, int g, wy_rows<IO, D, LP> &r,
                                                raw4<IO> (&v)[C / 16][NVW], raw4<IO> (&w)[C / 16][NVW]) {
  constexpr int NK = D / 16, NB = C / 16;
  constexpr float LOG2E = 1.4426950408889634f;
  // waves whose column tiles lie past dv load no v, w (uniform per wave)
  constexpr bool ALL_OWNERS = (NB - 1) * NVW < NK;
  const int t = 16 * I + m;
  const bool valid = t < len;
  const size_t row = static_cast<size_t>(t0 + (valid ? t : 0)) * a.H + h;
  const IO *bp = static_cast<const IO *>(a.b);
  const IO *ap = static_cast<const IO *>(a.al);
  const float *ga = static_cast<const float *>(a.al);
  if constexpr (SB)
    r.b[0] = raw4<IO>::first(bp[row]);
  if constexpr (SA && !LP)
    r.al[0] = raw4<IO>::first(ap[row]);
  if constexpr (SA && LP)
    r.lg[0][0] = ga[row];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const int c0 = 16 * kk + 4 * g;
    r.q[kk] = raw4<IO>::ld(static_cast<const IO *>(a.q) + row * D + c0);
    r.k[kk] = raw4<IO>::ld(static_cast<const IO *>(a.k) + row * D + c0);
    if constexpr (!SB)
      r.b[kk] = raw4<IO>::ld(bp + row * D + c0);
    if constexpr (!SA && !LP)
      r.al[kk] = raw4<IO>::ld(ap + row * D + c0);
    if constexpr (!SA && LP)
      r.lg[kk] = *reinterpret_cast<const f32x4 *>(ga + row * D + c0);
  }
  bool vjs[NB];
  if (ALL_OWNERS || owner) {
#pragma unroll
    for (int J = 0; J < NB; ++J) {
      const int tj = 16 * J + m;
      vjs[J] = tj < len;
      const size_t vrow = static_cast<size_t>(t0 + (vjs[J] ? tj : 0)) * a.H + h;
      if constexpr (SW)
        w[J][0] = raw4<IO>::first(static_cast<const IO *>(a.w)[vrow]);
#pragma unroll
      for (int j = 0; j < NVW; ++j) {
        const int c0 = 16 * (vt0 + j) + 4 * g;
        v[J][j] = raw4<IO>::ld(static_cast<const IO *>(a.v) + vrow * D + c0);
        if constexpr (!SW)
          w[J][j] = raw4<IO>::ld(static_cast<const IO *>(a.w) + vrow * D + c0);
      }
    }
  } else {
#pragma unroll
    for (int J = 0; J < NB; ++J) {
      vjs[J] = false;
#pragma unroll
      for (int j = 0; j < NVW; ++j)
        v[J][j] = w[J][j] = raw4<IO>::fill(0.f);
    }
  }
  // every load has issued; now the masks and splats
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
    r.k[kk] = raw4<IO>::select(valid, r.k[kk], 0.f);
  if constexpr (SB) {
    const raw4<IO> bs = raw4<IO>::splat(r.b[0].first());
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      r.b[kk] = bs;
  }
  if constexpr (!LP) {
    if constexpr (SA) {
      const raw4<IO> as = raw4<IO>::splat(valid ? r.al[0].first() : io<IO>::from_f(1.f));
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        r.al[kk] = as;
    } else {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        r.al[kk] = raw4<IO>::select(valid, r.al[kk], 1.f);
    }
  } else {
    if constexpr (SA) {
      const float gs = valid ? r.lg[0][0] * LOG2E : 0.f;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        r.lg[kk] = f32x4{gs, gs, gs, gs};
    } else {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        r.lg[kk] = valid ? r.lg[kk] * LOG2E : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int J = 0; J < NB; ++J) {
    if constexpr (SW) {
      const raw4<IO> s = raw4<IO>::splat(w[J][0].first());
#pragma unroll
      for (int j = 0; j < NVW; ++j)
        w[J][j] = s;
    }
#pragma unroll
    for (int j = 0; j < NVW; ++j)
      v[J][j] = raw4<IO>::select(vjs[J], v[J][j], 0.f);
  }
}

// Inputs of one chunk in input mode GM.  The modes that read the layouts at
// run time branch once, uniformly, into the straight-line variants.
template <typename IO, int D, int C, int NVW, int GM>
__device__ __forceinline__ void wy_load_chunk(const chunk_args &a, long t0, int len, int h, int I, int vt0,
                                              bool owner, int m, int g, wy_rows<IO, D, GM == GM_LAYER> &r,
                                              raw4<IO> (&v)[C / 16][NVW], raw4<IO> (&w)[C / 16][NVW]) {
  constexpr bool LP = GM == GM_LAYER;
#define GDN2_LOAD(SB, SW, SA) \
  wy_load_chunk_t<IO, D, C, NVW, LP, SB, SW, SA>(a, t0, len, h, I, vt0, owner, m, g, r, v, w)
  if constexpr (GM == GM_PLAIN) {
    GDN2_LOAD(false, false, false);
  } else if constexpr (GM == GM_KDA) {
    GDN2_LOAD(true, true, false);
  } else if constexpr (GM == GM_GDN) {
    GDN2_LOAD(true, true, true);
  } else {
    switch (a.gates & (GATE_SCALAR_B | GATE_SCALAR_W | GATE_SCALAR_ALPHA)) {
      case 0: GDN2_LOAD(false, false, false); break;
      case GATE_SCALAR_B: GDN2_LOAD(true, false, false); break;
      case GATE_SCALAR_W: GDN2_LOAD(false, true, false); break;
      case GATE_SCALAR_B | GATE_SCALAR_W: GDN2_LOAD(true, true, false); break;
      case GATE_SCALAR_ALPHA: GDN2_LOAD(false, false, true); break;
      case GATE_SCALAR_B | GATE_SCALAR_ALPHA: GDN2_LOAD(true, false, true); break;
      case GATE_SCALAR_W | GATE_SCALAR_ALPHA: GDN2_LOAD(false, true, true); break;
      default: GDN2_LOAD(true, true, true); break;
    }
  }
#undef GDN2_LOAD
}

// Decay over a sub-block below 2^-DIAG_LIM (in some channel) sends that
// sub-block's diagonal A and P blocks to the pairwise path.
constexpr float DIAG_LIM = 64.f;

// Value of lane m - J of this lane's DPP row (lanes 16g .. 16g+15), zero for
// m < J (row_shr:J).
template <int J> __device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + J, 0xF, 0xF, false));
}
// Value of lane m + J of this lane's DPP row, zero for m + J > 15 (row_shl:J).
template <int J> __device__ __forceinline__ float row_shl(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x100 + J, 0xF, 0xF, false));
}
// Sum of x over the lanes after this one in its DPP row (an exclusive
// suffix scan over the 16 tokens of a sub-block).
__device__ __forceinline__ float row16_exclusive_suffix(float x) {
  x = row_shl<1>(x);
  x += row_shl<1>(x);
  x += row_shl<2>(x);
  x += row_shl<4>(x);
  x += row_shl<8>(x);
  return x;
}

__device__ __forceinline__ float dot4(f32x4 x, f32x4 y) { return (x[0] * y[0] + x[1] * y[1]) + (x[2] * y[2] + x[3] * y[3]); }

// Row `row` ((token, head) index) of the inputs, this lane's channels
// c0 .. c0+3, as the recurrence's float32 values: q and k (times the row
// scales qs, ks: the L2 normalisation under layer prep, else 1), e = b (.) k
// and alpha itself.  Gate layouts and layer prep are read from a.gates.  An
// invalid row gives k = 0 and alpha = 1.
template <typename IO, int D>
__device__ __forceinline__ void wy_row4(const chunk_args &a, size_t row, bool valid, int c0, float qs, float ks,
                                        f32x4 &q4, f32x4 &k4, f32x4 &e4, f32x4 &a4) {
  constexpr float LOG2E = 1.4426950408889634f;
  const IO *bp = static_cast<const IO *>(a.b);
  const bool lp = (a.gates & GATE_LAYER_PREP) != 0, sa = (a.gates & GATE_SCALAR_ALPHA) != 0;
  q4 = io<IO>::load4(static_cast<const IO *>(a.q) + row * D + c0) * qs;
  k4 = io<IO>::load4(static_cast<const IO *>(a.k) + row * D + c0) * ks;
  f32x4 b4;
  if (a.gates & GATE_SCALAR_B) {
    const float x = io<IO>::to_f(bp[row]);
    b4 = f32x4{x, x, x, x};
  } else {
    b4 = io<IO>::load4(bp + row * D + c0);
  }
  if (lp) {
    const float *lg = static_cast<const float *>(a.al);
    const f32x4 l = sa ? f32x4{lg[row], lg[row], lg[row], lg[row]} : *reinterpret_cast<const f32x4 *>(lg + row * D + c0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b4[i] = fast_sigmoid(b4[i]);
      a4[i] = fast_exp2(l[i] * LOG2E);
    }
  } else if (sa) {
    const float x = io<IO>::to_f(static_cast<const IO *>(a.al)[row]);
    a4 = f32x4{x, x, x, x};
  } else {
    a4 = io<IO>::load4(static_cast<const IO *>(a.al) + row * D + c0);
  }
  if (!valid) {
    k4 = f32x4{0.f, 0.f, 0.f, 0.f};
    a4 = f32x4{1.f, 1.f, 1.f, 1.f};
  }
  e4 = b4 * k4;
}

// log2(alpha) of this lane's row (token 16 I + m of the chunk at t0, head h)
// for channels c0 .. c0+3, read again from global memory (layouts and layer
// prep from a.gates); rows past the end give 0.
template <typename IO, int D>
__device__ __forceinline__ f32x4 wy_log_decay4(const chunk_args &a, long t0, int len, int h, int I, int lane,
                                               int c0) {
  constexpr float LOG2E = 1.4426950408889634f;
  const int t = 16 * I + (lane & 15);
  const bool valid = t < len;
  const size_t row = static_cast<size_t>(t0 + (valid ? t : 0)) * a.H + h;
  const bool sa = (a.gates & GATE_SCALAR_ALPHA) != 0;
  f32x4 x;
  if (a.gates & GATE_LAYER_PREP) {
    const float *lg = static_cast<const float *>(a.al);
    x = sa ? f32x4{lg[row], lg[row], lg[row], lg[row]} : *reinterpret_cast<const f32x4 *>(lg + row * D + c0);
    x *= LOG2E;
  } else {
    const IO *ap = static_cast<const IO *>(a.al);
    const f32x4 al = sa ? f32x4{io<IO>::to_f(ap[row]), io<IO>::to_f(ap[row]), io<IO>::to_f(ap[row]),
                                io<IO>::to_f(ap[row])}
                        : io<IO>::load4(ap + row * D + c0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = fast_log2(al[i]);
  }
  return valid ? x : f32x4{0.f, 0.f, 0.f, 0.f};
}

// The diagonal A and P blocks of sub-block I, pair by pair:
//   A[t][s] = sum_c x_tc y_sc prod_{u=s+1..t} alpha_uc  (s < t),
//   P[t][s] = sum_c q_tc y_sc prod_{u=s+1..t} alpha_uc  (s <= t),
// with (x, y) = (e, k) for the default rule (SEL 0), (k, e) for the rule-R1
// erase products (SEL 1) and (k, k) for its write products (SEL 2),
// with the decay a running product of the alphas, so that any decay (alpha
// = 0 included) is exact to rounding.  The inputs are read again from
// global memory, one tile of 16 channels at a time; lane (t, g) walks the
// distances J = t - s in a loop, taking row t - J's values from the lane
// J below it in its 16-lane row.  Returns the blocks in the accumulator
// layout of the matrix-core product (lane (t, g) holds columns
// s = 4g .. 4g+3 of row t), zero outside the triangles.  A slow path: the
// loops are kept rolled so that it adds few registers to its kernel.
template <typename IO, int D, int SEL = 0>
__device__ __forceinline__ void wy_diag_pairwise(const chunk_args &a, long t0, int len, int h, int I, int lane,
                                                 float qs, float ks, f32x4 &dA, f32x4 &dP) {
  constexpr int NK = D / 16;
  const int m = lane & 15, g = lane >> 4, t = 16 * I + m;
  const bool valid = t < len;
  const size_t row = static_cast<size_t>(t0 + (valid ? t : 0)) * a.H + h;
  dA = dP = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int kk = 0; kk < NK; ++kk) {
    f32x4 q4, k4, e4, a4;
    wy_row4<IO, D>(a, row, valid, 16 * kk + 4 * g, qs, ks, q4, k4, e4, a4);
    const f32x4 x4 = SEL == 0 ? e4 : k4, y4 = SEL == 1 ? e4 : k4;
    f32x4 F = {1.f, 1.f, 1.f, 1.f};
#pragma unroll 1
    for (int J = 0; J < 16; ++J) {
      // F = alpha_t .. alpha_{t-J+1}; the key of row t - J
      const int src = m >= J ? lane - J : lane;
      const int srca = m >= J ? lane - J + 1 : lane;
      f32x4 kf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (J > 0)
          F[i] *= __shfl(a4[i], srca, 64);
        kf[i] = __shfl(y4[i], src, 64) * F[i];
      }
      float xa = m >= J ? dot4(x4, kf) : 0.f;
      float xp = m >= J ? dot4(q4, kf) : 0.f;
      xa += __shfl_xor(xa, 16, 64);
      xp += __shfl_xor(xp, 16, 64);
      xa += __shfl_xor(xa, 32, 64);
      xp += __shfl_xor(xp, 32, 64);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (m - (4 * g + i) == J) {
          if (J > 0)
            dA[i] += xa;
          dP[i] += xp;
        }
      }
    }
  }
}

// Layer prep: 1 / ||q_t|| and 1 / ||k_t|| of this lane's row (zero rows keep
// zero).  The lane holds 4 of every 16 channels; lanes m, m+16, m+32, m+48
// together hold the whole row.  Kept apart from the loads so that waiting for
// q and k does not hold back the loads issued after them.
template <typename IO, int D>
__device__ __forceinline__ void wy_row_scales(const wy_rows<IO, D, true> &r, float &qs, float &ks) {
  constexpr int NK = D / 16;
  float sq = 0.f, sk = 0.f;
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const f32x4 x = r.q[kk].f(), y = r.k[kk].f();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sq += x[i] * x[i];
      sk += y[i] * y[i];
    }
  }
  sq += __shfl_xor(sq, 16, 64);
  sk += __shfl_xor(sk, 16, 64);
  sq += __shfl_xor(sq, 32, 64);
  sk += __shfl_xor(sk, 32, 64);
  qs = sq > 0.f ? __frsqrt_rn(sq) : 0.f;
  ks = sk > 0.f ? __frsqrt_rn(sk) : 0.f;
}

// Phase 1: log2(alpha), prefix sums over the tokens of each sub-block, and the
// per-channel factors between sub-block boundaries.  On return gl holds the
// in-sub-block prefix sums g_t - rho_I, and pw is true (the same on every
// lane of the wave) when sub-block I's decay in some channel is below
// 2^-DIAG_LIM: its diagonal blocks then take the pairwise path
// (wy_diag_pairwise, on the inputs of the chunk at t0, len, head h, read
// again from a), which writes them to LDS where wy_products would.  gam_out[c] = gamma_C (may be LDS or
// global memory).  Contains two workgroup barriers.
template <typename IO, int D, int C, bool LP = false, int SEL = 0>
__device__ __forceinline__ void wy_decay(wy_smem<IO, D, C> &sm, const wy_rows<IO, D, LP> &r, f32x4 (&gl)[D / 16],
                                         bool &pw, const chunk_args &a, long t0, int len, int h, int I, int tid,
                                         float *gam_out) {
  constexpr int NB = C / 16, NK = D / 16;
  const int lane = tid & 63, m = lane & 15, g = lane >> 4;
  float mn = 0.f;
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    f32x4 x;
    if constexpr (LP) {
      x = r.lg[kk];
    } else {
      const f32x4 al = r.al[kk].f();
#pragma unroll
      for (int i = 0; i < 4; ++i)
        x[i] = fast_log2(al[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gl[kk][i] = row16_inclusive_scan(x[i]);
      mn = fminf(mn, gl[kk][i]);
    }
  }
  pw = __ballot(m == 15 && mn < -DIAG_LIM) != 0;
  if (pw) {
    // the diagonal A and P blocks go straight to where the products would
    // put them (wy_products skips them)
    float qs = 1.f, ks = 1.f;
    if constexpr (LP)
      wy_row_scales<IO, D>(r, qs, ks);
    f32x4 da, dp;
    wy_diag_pairwise<IO, D, SEL>(a, t0, len, h, I, lane, qs, ks, da, dp);
    *reinterpret_cast<f32x4 *>(&sm.ad[I][m][4 * g]) = da;
    frag<IO>::from(dp).st(sm.pr[tri_index(I, I)], lane);
  }
  if (m == 15) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      *reinterpret_cast<f32x4 *>(&sm.tot[I][16 * kk + 4 * g]) = gl[kk];
  }
  __syncthreads();
  for (int idx = tid; idx < NB * D; idx += 64 * NB) {
    const int J = idx / D, c = idx - J * D;
    float rho = 0.f, suf = 0.f, all = 0.f;
#pragma unroll
    for (int K = 0; K < NB; ++K) {
      const float x = sm.tot[K][c];
      all += x;
      if (K < J)
        rho += x;
      else if (K > J)
        suf += x;
    }
    sm.f1[J][c] = fast_exp2(rho);
    sm.f2[J][c] = fast_exp2(suf);
    float part = 0.f;  // sum of tot over sub-blocks J+1 .. I2-1
#pragma unroll
    for (int I2 = 1; I2 < NB; ++I2) {
      if (I2 > J) {
        sm.sig[pair_index(I2, J)][c] = fast_exp2(part);
        part += sm.tot[I2][c];
      }
    }
    if (J == 0)
      gam_out[c] = fast_exp2(all);
  }
  __syncthreads();
}

// Register operands of the A and P products for sub-block I.  With pw the
// diagonal blocks are already in LDS (wy_decay).
template <typename IO, int D> struct wy_ops {
  static constexpr int NK = D / 16;
  frag<IO> ef[NK], qf[NK], khf[NK], qcf[NK];
  bool pw;
};

// Phase 1b: decayed, gated operands of sub-block I.  Writes the rescaled keys
// for later sub-blocks and ColFrag(E) to LDS, and RowFrag(Kbar^T) tiles to
// kb_out (the KB region of a block layout, LDS or global).  With pw (from
// wy_decay) the key suffixes are read again from the chunk's inputs (chunk
// t0, len, head h of a).
template <typename IO, int D, int C, bool LP = false>
__device__ __forceinline__ void wy_operands(wy_smem<IO, D, C> &sm, const wy_rows<IO, D, LP> &r,
                                            const f32x4 (&gl)[D / 16], bool pw, const chunk_args &a, long t0,
                                            int len, int h, int I, int lane,
                                            const frag<IO> &eye, unsigned char *kb_out, wy_ops<IO, D> &op) {
  constexpr int NB = C / 16, NK = D / 16;
  typedef frag<IO> F;
  const int g = lane >> 4;
  float qs = 1.f, ks = 1.f;
  if constexpr (LP)
    wy_row_scales<IO, D>(r, qs, ks);
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const int c0 = 16 * kk + 4 * g;
    const f32x4 f1v = *reinterpret_cast<const f32x4 *>(&sm.f1[I][c0]);
    const f32x4 f2v = *reinterpret_cast<const f32x4 *>(&sm.f2[I][c0]);
    // suffix rho_{I+1} - g_t of the log decay within the sub-block: the
    // sub-block's total minus the prefix while both are bounded, else the
    // suffix scan of the log decays themselves (read again)
    f32x4 sfx;
    if (!pw) {
      sfx = *reinterpret_cast<const f32x4 *>(&sm.tot[I][c0]) - gl[kk];
    } else {
      const f32x4 x = wy_log_decay4<IO, D>(a, t0, len, h, I, lane, c0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sfx[i] = row16_exclusive_suffix(x[i]);
    }
    f32x4 f, fk, fi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = fast_exp2(gl[kk][i]);                  // e^{g_t - rho_I} <= 1
      fk[i] = fast_exp2(sfx[i]);                    // e^{rho_{I+1} - g_t} <= 1
      fi[i] = pw ? 0.f : fast_exp2(-gl[kk][i]);     // e^{rho_I - g_t} <= 2^64 (diagonal product only)
    }
    f32x4 kf = r.k[kk].f(), bf = r.b[kk].f(), qf = r.q[kk].f();
    if constexpr (LP) {
      kf *= ks;
      qf *= qs;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bf[i] = fast_sigmoid(bf[i]);
    }
    const f32x4 er = bf * kf * f;
    const f32x4 qr = qf * f;
    const f32x4 kt = kf * fk;
    op.ef[kk] = F::from(er);
    op.qf[kk] = F::from(qr);
    op.khf[kk] = F::from(kf * fi);
    op.qcf[kk] = F::from(qr * f1v);
    // keys of this sub-block referenced to the start of each later one
#pragma unroll
    for (int I2 = 1; I2 < NB; ++I2) {
      if (I2 > I) {
        const f32x4 s = *reinterpret_cast<const f32x4 *>(&sm.sig[pair_index(I2, I)][c0]);
        F::from(kt * s).st(&sm.khs[pair_index(I2, I)][0][0] + tile_off<IO, NK>(0, kk, lane), 0);
      }
    }
    F::from(transpose_frag(F::from(er * f1v), eye)).st(sm.ec[I][kk], lane);
    F::from(transpose_frag(F::from(kt * f2v), eye)).st(kb_out + tile_off<IO, NB>(kk, I, lane), 0);
  }
  op.pw = pw;
}

// ColFrag(U_J) = ColFrag(w (.) v) for NVW column tiles and every sub-block.
template <typename IO, int NB, int NVW, bool LP = false>
__device__ __forceinline__ void wy_values(const raw4<IO> (&v)[NB][NVW], const raw4<IO> (&w)[NB][NVW],
                                          const frag<IO> &eye, frag<IO> (&ucol)[NB][NVW]) {
#pragma unroll
  for (int J = 0; J < NB; ++J)
#pragma unroll
    for (int j = 0; j < NVW; ++j) {
      f32x4 wf = w[J][j].f();
      if constexpr (LP) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          wf[i] = fast_sigmoid(wf[i]);
      }
      ucol[J][j] = frag<IO>::from(transpose_frag(frag<IO>::from(wf * v[J][j].f()), eye));
    }
}

// Phase 2: A and P rows of sub-block I.  RowFrag(A_IK) stays in registers
// (af), RowFrag(P_IJ) and the diagonal A block go to LDS.  Ends with a
// barrier, after which RowFrag(Qchk) replaces the rescaled keys in LDS.
template <typename IO, int D, int C>
__device__ __forceinline__ void wy_products(wy_smem<IO, D, C> &sm, const wy_ops<IO, D> &op, int I, int lane,
                                            frag<IO> (&af)[C / 16]) {
  constexpr int NB = C / 16, NK = D / 16;
  typedef frag<IO> F;
  typedef frag2<IO> F2;
  const int m = lane & 15, g = lane >> 4;
  f32x4 accA[NB], accP[NB];
#pragma unroll
  for (int J = 0; J < NB; ++J) {
    accA[J] = f32x4{0.f, 0.f, 0.f, 0.f};
    accP[J] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (J < I) {
      const unsigned char *kb = &sm.khs[pair_index(I, J)][0][0];
      if constexpr (NK % 2 == 0) {
#pragma unroll
        for (int kp = 0; kp < NK / 2; ++kp) {
          const F2 a2 = F2::ld(kb + tile_off<IO, NK>(0, 2 * kp, 0), lane);
          mma32(accA[J], a2, F2::make(op.ef[2 * kp], op.ef[2 * kp + 1]));
          mma32(accP[J], a2, F2::make(op.qf[2 * kp], op.qf[2 * kp + 1]));
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const F a1 = F::ld(kb + tile_off<IO, NK>(0, kk, 0), lane);
          mma16(accA[J], a1, op.ef[kk]);
          mma16(accP[J], a1, op.qf[kk]);
        }
      }
    } else if (J == I && !op.pw) {
      if constexpr (NK % 2 == 0) {
#pragma unroll
        for (int kp = 0; kp < NK / 2; ++kp) {
          const F2 a2 = F2::make(op.khf[2 * kp], op.khf[2 * kp + 1]);
          mma32(accA[J], a2, F2::make(op.ef[2 * kp], op.ef[2 * kp + 1]));
          mma32(accP[J], a2, F2::make(op.qf[2 * kp], op.qf[2 * kp + 1]));
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          mma16(accA[J], op.khf[kk], op.ef[kk]);
          mma16(accP[J], op.khf[kk], op.qf[kk]);
        }
      }
      // lane (t = m, g) holds row t, columns s = 4g + i of the diagonal block
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!(4 * g + i < m))
          accA[J][i] = 0.f;
        if (!(4 * g + i <= m))
          accP[J][i] = 0.f;
      }
      *reinterpret_cast<f32x4 *>(&sm.ad[I][m][4 * g]) = accA[J];
    }
    if (J < I || (J == I && !op.pw))
      F::from(accP[J]).st(sm.pr[tri_index(I, J)], lane);
  }
#pragma unroll
  for (int K = 0; K < NB; ++K)
    af[K] = F::from(accA[K]);
  __syncthreads();
  unsigned char *qc_tiles = &sm.khs[0][0][0];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
    op.qcf[kk].st(qc_tiles + (I * NK + kk) * wy_smem<IO, D, C>::TB, lane);
}

// Phase 3: T = (I + A)^{-1} into LDS (ColFrag and RowFrag of every block).
// Contains NB workgroup barriers; the last one publishes all of T.
template <typename IO, int D, int C>
__device__ __forceinline__ void wy_inverse(wy_smem<IO, D, C> &sm, const frag<IO> (&af)[C / 16], int I, int lane,
                                           const frag<IO> &eye) {
  constexpr int NB = C / 16;
  typedef frag<IO> F;
  const int m = lane & 15, g = lane >> 4;
  {
    // diagonal block: lane column c = m, rows kept: 4g .. 4g+3
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = (i == m) ? 1.f : 0.f;
#pragma unroll
      for (int j = 0; j < i; ++j)
        acc -= sm.ad[I][i][j] * x[j];
      x[i] = acc;
    }
    f32x4 tii;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      tii[i] = (g == 0) ? x[i] : (g == 1) ? x[4 + i] : (g == 2) ? x[8 + i] : x[12 + i];
    const F tf = F::from(tii);
    tf.st(sm.tcol[tri_index(I, I)], lane);
    F::from(transpose_frag(tf, eye)).st(sm.trow[tri_index(I, I)], lane);
  }
  __syncthreads();
  if constexpr (NB > 1) {
    const F trow_ii = F::ld(sm.trow[tri_index(I, I)], lane);
#pragma unroll
    for (int l = 1; l < NB; ++l) {
      if (I >= l) {
        const int J = I - l;
        F tk[NB];
#pragma unroll
        for (int K = 0; K < NB; ++K)
          tk[K] = (K >= J && K < I) ? F::ld(sm.tcol[tri_index(K, J)], lane) : F::zero();
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int K = 0; K < NB; ++K)
          if (K >= J && K < I)
            mma16(acc, af[K], tk[K]);
        f32x4 tij = {0.f, 0.f, 0.f, 0.f};
        mma16(tij, trow_ii, F::from(acc));
        const F tf = F::from(-tij);
        tf.st(sm.tcol[tri_index(I, J)], lane);
        F::from(transpose_frag(tf, eye)).st(sm.trow[tri_index(I, J)], lane);
      }
      __syncthreads();
    }
  }
}

// T and P tiles of a chunk, loaded once by every wave for phases 4-5 (all
// operand loads are issued before the products that use them).
template <typename IO, int C> struct wy_tp {
  static constexpr int NT = (C / 16) * (C / 16 + 1) / 2;
  frag<IO> tr[NT];  // RowFrag(T_IJ)
  frag<IO> p[NT];   // RowFrag(P_IJ)
};

template <typename IO, int D, int C>
__device__ __forceinline__ void wy_load_tp(const wy_smem<IO, D, C> &sm, int lane, wy_tp<IO, C> &tp) {
#pragma unroll
  for (int i = 0; i < wy_tp<IO, C>::NT; ++i) {
    tp.tr[i] = frag<IO>::ld(sm.trow[i], lane);
    tp.p[i] = frag<IO>::ld(sm.pr[i], lane);
  }
}

// Phases 4-5 for one dk column tile ct: W = T E and Q' = Qchk - P W (the latter
// computed as Q'^T = Qchk^T - W^T P^T so that it lands as RowFrag).  Writes
// RowFrag(-W) and RowFrag(Q') tiles to wn_out / qp_out (block layout, LDS or
// global, k tiles paired).
template <typename IO, int D, int C>
__device__ __forceinline__ void wy_wq(const wy_smem<IO, D, C> &sm, const wy_tp<IO, C> &tp, int ct, int lane,
                                      const frag<IO> &eye, unsigned char *__restrict__ wn_out,
                                      unsigned char *__restrict__ qp_out) {
  constexpr int NB = C / 16, NK = D / 16;
  typedef frag<IO> F;
  const unsigned char *qc_tiles = &sm.khs[0][0][0];
  F ecf[NB], qcf[NB];
#pragma unroll
  for (int J = 0; J < NB; ++J) {
    ecf[J] = F::ld(sm.ec[J][ct], lane);
    qcf[J] = F::ld(qc_tiles + (J * NK + ct) * wy_smem<IO, D, C>::TB, lane);
  }
  F wc[NB];
#pragma unroll
  for (int I2 = 0; I2 < NB; ++I2) {
    f32x4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J <= I2; ++J)
      mma16(w, tp.tr[tri_index(I2, J)], ecf[J]);
    wc[I2] = F::from(w);
  }
#pragma unroll
  for (int I2 = 0; I2 < NB; ++I2) {
    f32x4 q = qcf[I2].to_f32();
#pragma unroll
    for (int J = 0; J <= I2; ++J)
      mma16(q, wc[J], tp.p[tri_index(I2, J)].neg());
    F::from(transpose_frag(wc[I2], eye)).neg().st(wn_out + tile_off<IO, NK>(I2, ct, lane), 0);
    F::from(q).st(qp_out + tile_off<IO, NK>(I2, ct, lane), 0);
  }
}

// Phases 4-5 for one dv column tile: Ut = T U and O_intra = P Ut, returned as
// float accumulators (ut[I], oi[I] for the 16 rows of sub-block I).  ut is
// ColFrag; oi is ColFrag, or RowFrag when OI_ROW (computed as O_intra^T =
// Ut^T P^T by swapping the operands, which puts 4 consecutive columns of one
// row in each lane).  Without WITH_O only Ut is formed (oi untouched).
template <typename IO, int C, bool OI_ROW = false, bool WITH_O = true>
__device__ __forceinline__ void wy_uo(const wy_tp<IO, C> &tp, const frag<IO> (&ucol)[C / 16],
                                      f32x4 (&ut)[C / 16], f32x4 (&oi)[C / 16]) {
  constexpr int NB = C / 16;
  typedef frag<IO> F;
  F uc[NB];
#pragma unroll
  for (int I2 = 0; I2 < NB; ++I2) {
    f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J <= I2; ++J)
      mma16(u, tp.tr[tri_index(I2, J)], ucol[J]);
    ut[I2] = u;
    uc[I2] = F::from(u);
  }
  if constexpr (!WITH_O)
    return;
#pragma unroll
  for (int I2 = 0; I2 < NB; ++I2) {
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J <= I2; ++J) {
      if constexpr (OI_ROW)
        mma16(o, uc[J], tp.p[tri_index(I2, J)]);
      else
        mma16(o, tp.p[tri_index(I2, J)], uc[J]);
    }
    oi[I2] = o;
  }
}

}  // namespace gdn2
