// gdn2_rule_r1.hip -- the chunked two-pass forward of reading R1 (gfx950).
//
// Reading R1 of the pages' formal paragraph (aixai.ru blog, section on why
// one scalar cannot serve both decisions) erases along the gated key and
// reads with the key itself:
//   D = Diag(alpha_t) S;  r_t = D^T k_t;  S_t = D - e_t r_t^T + k_t u_t^T,
// e = b (.) k, u = w (.) v, o_t = S_t^T q_t.  Its erase and its write have
// different left vectors, so a chunk carries the reads R = [r_t] as well as
// the writes.  With g the cumulative log decay from the chunk start and
// Kchk = k e^g, Ehat = e e^-g, Khat = k e^-g, Qchk = q e^g (per channel):
//   (I + A') R = Kchk S0 + B' U,  A' = strict_lower(Kchk Ehat^T),
//   B' = strict_lower(Kchk Khat^T),  T' = (I + A')^-1,
//   R  = W' S0 + Ut',  W' = T' Kchk,  Ut' = T' B' U,
//   O  = (Qchk - P_e W') S0 + (P_k U - P_e Ut'),
//        P_e = lower(Qchk Ehat^T),  P_k = lower(Qchk Khat^T),
//   S_C = Diag(gamma_C) S0 - Ebar^T R + Kbar^T U,
//        Ebar = e e^{g_C - g},  Kbar = k e^{g_C - g}.
// The products with Ehat keys are the default rule's with the roles of e and
// k swapped, so the per-chunk phases of gdn2_wy.hpp compute A', P_e, T', W'
// and Q'' = Qchk - P_e W' unchanged once the operands are swapped; this file
// adds the products with Khat keys (B', P_k), Ut' and O'' = P_k U - P_e Ut',
// and N = Kbar^T U.  The block stores -W', Q'', Ebar^T, gamma_C, -Ut', O''
// and N, so that the state scan is the default rule's with Z = -R and one
// more term:  Z = -Ut' - W' S,  O = Q'' S + O'',  S <- Diag(gamma) S +
// Ebar^T Z + N.  Every decay factor is formed as in gdn2_wy.hpp (sums of log
// decays, pairwise diagonal blocks under strong decay).
#include "gdn2_wy.hpp"

namespace gdn2 {

template <typename IO, int D, int C> size_t r1_block_bytes() { return r1_layout<IO, D, C>::BYTES; }

// LDS of the rule-R1 products beyond wy_smem: the Khat keys of each later
// sub-block, the B' and P_k tiles and RowFrag(Kbar^T) for N.
template <typename IO, int D, int C> struct r1_smem {
  static constexpr int NB = C / 16, NK = D / 16;
  static constexpr int NP = NB * (NB - 1) / 2, NT = NB * (NB + 1) / 2;
  static constexpr int NKS = (NP > 0 ? NP : 1);
  static constexpr int TB = frag<IO>::TILE_BYTES;
  alignas(16) unsigned char khs2[NKS][NK][TB];  // RowFrag(k_s e^{rho_I - g_s}) for pair (I, J), J < I
  alignas(16) unsigned char bp[NT][TB];         // RowFrag(B'_IJ)
  alignas(16) unsigned char pk[NT][TB];         // RowFrag(P_k,IJ)
  alignas(16) unsigned char kbar[NK][NB][TB];   // RowFrag(Kbar^T) tile (kk, tt), paired as tile_off<NB>
};

// Operands of sub-block I for rule R1: rows Kchk (in op.ef), Qchk; keys Ehat
// (LDS khs, op.khf for the diagonal) and Khat (r1 khs2, khf2); E slot of the
// W product = Kchk; the KB slot of the block = Ebar^T, and Kbar^T to LDS.
template <typename IO, int D, int C, bool LP>
__device__ __forceinline__ void r1_operands(wy_smem<IO, D, C> &sm, r1_smem<IO, D, C> &sx,
                                            const wy_rows<IO, D, LP> &r, const f32x4 (&gl)[D / 16], bool pw,
                                            const chunk_args &a, long t0, int len, int h, int I, int lane,
                                            const frag<IO> &eye, unsigned char *kb_out, wy_ops<IO, D> &op,
                                            frag<IO> (&khf2)[D / 16]) {
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
      f[i] = fast_exp2(gl[kk][i]);
      fk[i] = fast_exp2(sfx[i]);
      fi[i] = pw ? 0.f : fast_exp2(-gl[kk][i]);
    }
    f32x4 kf = r.k[kk].f(), bf = r.b[kk].f(), qf = r.q[kk].f();
    if constexpr (LP) {
      kf *= ks;
      qf *= qs;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bf[i] = fast_sigmoid(bf[i]);
    }
    const f32x4 ef = bf * kf;
    const f32x4 kr = kf * f, qr = qf * f;
    const f32x4 kte = ef * fk, ktk = kf * fk;  // keys to the end of their sub-block
    op.ef[kk] = F::from(kr);
    op.qf[kk] = F::from(qr);
    op.khf[kk] = F::from(ef * fi);
    khf2[kk] = F::from(kf * fi);
    op.qcf[kk] = F::from(qr * f1v);
#pragma unroll
    for (int I2 = 1; I2 < NB; ++I2) {
      if (I2 > I) {
        const f32x4 s = *reinterpret_cast<const f32x4 *>(&sm.sig[pair_index(I2, I)][c0]);
        F::from(kte * s).st(&sm.khs[pair_index(I2, I)][0][0] + tile_off<IO, NK>(0, kk, lane), 0);
        F::from(ktk * s).st(&sx.khs2[pair_index(I2, I)][0][0] + tile_off<IO, NK>(0, kk, lane), 0);
      }
    }
    F::from(transpose_frag(F::from(kr * f1v), eye)).st(sm.ec[I][kk], lane);
    F::from(transpose_frag(F::from(kte * f2v), eye)).st(kb_out + tile_off<IO, NB>(kk, I, lane), 0);
    F::from(transpose_frag(F::from(ktk * f2v), eye)).st(&sx.kbar[0][0][0] + tile_off<IO, NB>(kk, I, lane), 0);
  }
  op.pw = pw;
}

// A', P_e (as wy_products: af in registers, P_e and the diagonal of A' to LDS)
// and B', P_k (to LDS) for the rows of sub-block I.  With pw the diagonal
// blocks are formed pair by pair (A', P_e in wy_decay already).  Ends with a
// barrier, after which RowFrag(Qchk) replaces the Ehat keys in LDS.
template <typename IO, int D, int C>
__device__ __forceinline__ void r1_products(wy_smem<IO, D, C> &sm, r1_smem<IO, D, C> &sx, const wy_ops<IO, D> &op,
                                            const frag<IO> (&khf2)[D / 16], const chunk_args &a, long t0, int len,
                                            int h, float qs, float ks, int I, int lane, frag<IO> (&af)[C / 16]) {
  constexpr int NB = C / 16, NK = D / 16;
  typedef frag<IO> F;
  const int m = lane & 15, g = lane >> 4;
#pragma unroll
  for (int J = 0; J < NB; ++J) {
    f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = accA, accB = accA, accK = accA;
    if (J < I) {
      const unsigned char *ke = &sm.khs[pair_index(I, J)][0][0];
      const unsigned char *kk2 = &sx.khs2[pair_index(I, J)][0][0];
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const F ae = F::ld_at(ke + tile_off<IO, NK>(0, kk, lane));
        const F ak = F::ld_at(kk2 + tile_off<IO, NK>(0, kk, lane));
        mma16(accA, ae, op.ef[kk]);
        mma16(accP, ae, op.qf[kk]);
        mma16(accB, ak, op.ef[kk]);
        mma16(accK, ak, op.qf[kk]);
      }
    } else if (J == I) {
      if (!op.pw) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          mma16(accA, op.khf[kk], op.ef[kk]);
          mma16(accP, op.khf[kk], op.qf[kk]);
          mma16(accB, khf2[kk], op.ef[kk]);
          mma16(accK, khf2[kk], op.qf[kk]);
        }
      } else {
        wy_diag_pairwise<IO, D, 2>(a, t0, len, h, I, lane, qs, ks, accB, accK);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!(4 * g + i < m)) {
          accA[i] = 0.f;
          accB[i] = 0.f;
        }
        if (!(4 * g + i <= m)) {
          accP[i] = 0.f;
          accK[i] = 0.f;
        }
      }
      if (!op.pw)
        *reinterpret_cast<f32x4 *>(&sm.ad[I][m][4 * g]) = accA;
    }
    if (J < I || (J == I && !op.pw))
      F::from(accP).st(sm.pr[tri_index(I, J)], lane);
    if (J <= I) {
      F::from(accB).st(sx.bp[tri_index(I, J)], lane);
      F::from(accK).st(sx.pk[tri_index(I, J)], lane);
    }
    af[J] = F::from(accA);
  }
  __syncthreads();
  unsigned char *qc_tiles = &sm.khs[0][0][0];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
    op.qcf[kk].st(qc_tiles + (I * NK + kk) * wy_smem<IO, D, C>::TB, lane);
}

// For one dv column tile: V = B' U, Ut' = T' V, O''^T = U^T P_k^T - Ut'^T P_e^T
// (RowFrag(O'') in the accumulator), returned as -Ut' (ColFrag) and O''.
template <typename IO, int D, int C>
__device__ __forceinline__ void r1_uo(const wy_tp<IO, C> &tp, const r1_smem<IO, D, C> &sx, int lane,
                                      const frag<IO> (&ucol)[C / 16], frag<IO> (&utn)[C / 16],
                                      frag<IO> (&oi)[C / 16]) {
  constexpr int NB = C / 16;
  typedef frag<IO> F;
  F vf[NB];
#pragma unroll
  for (int I2 = 0; I2 < NB; ++I2) {
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J <= I2; ++J)
      mma16(v, F::ld(sx.bp[tri_index(I2, J)], lane), ucol[J]);
    vf[I2] = F::from(v);
  }
#pragma unroll
  for (int I2 = 0; I2 < NB; ++I2) {
    f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J <= I2; ++J)
      mma16(u, tp.tr[tri_index(I2, J)], vf[J]);
    utn[I2] = F::from(-u);
  }
#pragma unroll
  for (int I2 = 0; I2 < NB; ++I2) {
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int J = 0; J <= I2; ++J) {
      mma16(o, ucol[J], F::ld(sx.pk[tri_index(I2, J)], lane));
      mma16(o, utn[J], tp.p[tri_index(I2, J)]);
    }
    oi[I2] = F::from(o);
  }
}

// Pass 1 of rule R1.  grid: num_slots * H, block: 64 * C/16 threads.
template <typename IO, int D, int C, int GM>
__global__ void __launch_bounds__(64 * (C / 16)) gdn2_r1_prep_kernel(chunk_args a) {
  constexpr int NB = C / 16, NK = D / 16;
  constexpr int CTW = (NK >= NB) ? NK / NB : 1;  // column tiles per wave
  typedef frag<IO> F;
  typedef r1_layout<IO, D, C> R;
  typedef blk_layout<IO, D, C> L;
  __shared__ wy_smem<IO, D, C> sm;
  __shared__ r1_smem<IO, D, C> sx;

  const int h = blockIdx.x % a.H;
  const int slot = blockIdx.x / a.H;
  int seq, len;
  long t0;
  if (!locate_chunk<C>(slot, a, seq, t0, len))
    return;  // whole workgroup
  (void)seq;
  const int tid = threadIdx.x, I = tid >> 6, lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  (void)m;
  (void)g;
  const int ct0 = I * CTW;
  const bool owner = ct0 < NK;
  unsigned char *blk = reinterpret_cast<unsigned char *>(a.blocks) + (static_cast<size_t>(slot) * a.H + h) * a.blk_bytes;

  constexpr bool LP = GM == GM_LAYER;
  wy_rows<IO, D, LP> r;
  raw4<IO> rv[NB][CTW], rw[NB][CTW];
  wy_load_chunk<IO, D, C, CTW, GM>(a, t0, len, h, I, ct0, owner, m, g, r, rv, rw);
  f32x4 gl[NK];
  bool pw;
  wy_decay<IO, D, C, LP, 1>(sm, r, gl, pw, a, t0, len, h, I, tid, reinterpret_cast<float *>(blk + L::GAM));
  const F eye = identity_colfrag<IO>(lane);
  wy_ops<IO, D> op;
  F khf2[NK];
  r1_operands<IO, D, C, LP>(sm, sx, r, gl, pw, a, t0, len, h, I, lane, eye, blk + L::KB, op, khf2);
  float qs = 1.f, ks = 1.f;
  if constexpr (LP)
    wy_row_scales<IO, D>(r, qs, ks);
  F ucol[NB][CTW];
  wy_values<IO, NB, CTW, LP>(rv, rw, eye, ucol);
  __syncthreads();
  F af[NB];
  r1_products<IO, D, C>(sm, sx, op, khf2, a, t0, len, h, qs, ks, I, lane, af);
  wy_inverse<IO, D, C>(sm, af, I, lane, eye);
  if (owner) {
    wy_tp<IO, C> tp;
    wy_load_tp<IO, D, C>(sm, lane, tp);
#pragma unroll
    for (int j = 0; j < CTW; ++j) {
      const int ct = ct0 + j;
      wy_wq<IO, D, C>(sm, tp, ct, lane, eye, blk + L::WN, blk + L::QP);
      F uc_j[NB], utn[NB], oi[NB];
#pragma unroll
      for (int J = 0; J < NB; ++J)
        uc_j[J] = ucol[J][j];
      r1_uo<IO, D, C>(tp, sx, lane, uc_j, utn, oi);
#pragma unroll
      for (int I2 = 0; I2 < NB; ++I2) {
        utn[I2].st_at(blk + R::UT + tile_off<IO, NK>(I2, ct, lane));
        oi[I2].st_at(blk + R::OI + tile_off<IO, NK>(I2, ct, lane));
      }
      // N tile (kk, ct) = sum over the chunk's tokens of Kbar^T U
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        f32x4 n = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int tt = 0; tt < NB; ++tt)
          mma16(n, F::ld_at(&sx.kbar[0][0][0] + tile_off<IO, NB>(kk, tt, lane)), uc_j[tt]);
        F::from(n).st_at(blk + R::NC + tile_off<IO, NK>(kk, ct, lane));
      }
    }
  }
}

// Pass 2 of rule R1 where the scan kernel of gdn2_chunk.hip does not take
// it (float32, or an odd number of 16-wide tiles in D or C): the state scan
// with one wave per 16-column tile of the state (dk x 16 float32 in
// matrix-core accumulators), WPG waves per workgroup, every operand read
// from the block in global memory.  For chunk
// c: Z = -Ut' + (-W') S, O^T = S^T Q''^T + O''^T (stored as rows of four
// consecutive columns), S <- Diag(gamma_C) S + Ebar^T Z + N.
template <typename IO, int D, int C> struct r1_scan_cfg {
  static constexpr int NK = D / 16;
  static constexpr int WPG = NK < 4 ? NK : 4;  // waves (column tiles) per workgroup
  static constexpr int NGRP = NK / WPG;
};

template <typename IO, int D, int C>
__global__ void __launch_bounds__(64 * (r1_scan_cfg<IO, D, C>::WPG)) gdn2_r1_scan_kernel(chunk_args a) {
  constexpr int NB = C / 16, NK = D / 16, NGRP = r1_scan_cfg<IO, D, C>::NGRP, WPG = r1_scan_cfg<IO, D, C>::WPG;
  typedef frag<IO> F;
  typedef blk_layout<IO, D, C> L;
  typedef r1_layout<IO, D, C> R;
  const int unit = static_cast<int>(blockIdx.x) / NGRP, grp = static_cast<int>(blockIdx.x) % NGRP;
  if (unit >= a.num_seqs * a.H)
    return;
  const int n = unit / a.H, h = unit - n * a.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int j = grp * WPG + wave;  // this wave's dv tile
  int c_begin, nchunks;
  long tstart, tend;
  sequence_range<C>(n, a, c_begin, nchunks, tstart, tend);
  f32x4 S[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[kk][i] = a.S0 ? a.S0[(static_cast<size_t>(unit) * D + 16 * kk + 4 * g + i) * D + 16 * j + m] : 0.f;
  typedef __attribute__((address_space(1))) typename io<IO>::elem gelem;
  gelem *gout = (gelem *)(a.o);
  const unsigned char *blocks = reinterpret_cast<const unsigned char *>(a.blocks);
  for (int c = 0; c < nchunks; ++c) {
    const unsigned char *blk = blocks + (static_cast<size_t>(c_begin + c) * a.H + h) * a.blk_bytes;
    const long t0 = tstart + static_cast<long>(c) * C;
    const int len = (tend - t0) < C ? static_cast<int>(tend - t0) : C;
    F sf[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      sf[kk] = F::from(S[kk]);
    F zf[NB];
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
      f32x4 z = F::ld_at(blk + R::UT + tile_off<IO, NK>(tt, j, lane)).to_f32();
      f32x4 ot = F::ld_at(blk + R::OI + tile_off<IO, NK>(tt, j, lane)).to_f32();
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        mm_io(z, F::ld_at(blk + L::WN + tile_off<IO, NK>(tt, kk, lane)), sf[kk]);
        mm_io(ot, sf[kk], F::ld_at(blk + L::QP + tile_off<IO, NK>(tt, kk, lane)));
      }
      zf[tt] = F::from(z);
      const int t = 16 * tt + m;
      if (t < len)
        store4_global(gout + (static_cast<size_t>(t0 + t) * a.H + h) * D + 16 * j + 4 * g, ot);
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const f32x4 gm = *reinterpret_cast<const f32x4 *>(blk + L::GAM + (16 * kk + 4 * g) * sizeof(float));
      f32x4 s = S[kk] * gm + F::ld_at(blk + R::NC + tile_off<IO, NK>(kk, j, lane)).to_f32();
#pragma unroll
      for (int tt = 0; tt < NB; ++tt)
        mm_io(s, F::ld_at(blk + L::KB + tile_off<IO, NB>(kk, tt, lane)), zf[tt]);
      S[kk] = s;
    }
  }
  if (a.S_final) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a.S_final[(static_cast<size_t>(unit) * D + 16 * kk + 4 * g + i) * D + 16 * j + m] = S[kk][i];
  }
}

template <typename IO, int D, int C> hipError_t launch_r1_prep(const chunk_args &a, hipStream_t st) {
  if (a.num_slots == 0)
    return hipSuccess;
  const dim3 grid(static_cast<unsigned>(static_cast<long>(a.num_slots) * a.H)), block(64 * (C / 16));
  if (a.gates == 0)
    hipLaunchKernelGGL((gdn2_r1_prep_kernel<IO, D, C, GM_PLAIN>), grid, block, 0, st, a);
  else if (a.gates & GATE_LAYER_PREP)
    hipLaunchKernelGGL((gdn2_r1_prep_kernel<IO, D, C, GM_LAYER>), grid, block, 0, st, a);
  else  // per-(token, head) gates, read from the flags
    hipLaunchKernelGGL((gdn2_r1_prep_kernel<IO, D, C, GM_GATES>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <typename IO, int D, int C> hipError_t launch_r1_scan(const chunk_args &a, hipStream_t st) {
  if constexpr (scan_r1_supported<IO, D, C>()) {
    return launch_chunk_scan_r1<IO, D, C>(a, st);  // loader waves and LDS staging
  } else {
    typedef r1_scan_cfg<IO, D, C> K;
    const long units = static_cast<long>(a.num_seqs) * a.H;
    hipLaunchKernelGGL((gdn2_r1_scan_kernel<IO, D, C>), dim3(static_cast<unsigned>(units * K::NGRP)),
                       dim3(64 * K::WPG), 0, st, a);
    return hipGetLastError();
  }
}

#define GDN2_INST_R1(IO, D, C)                                                   \
  template size_t r1_block_bytes<IO, D, C>();                                   \
  template hipError_t launch_r1_prep<IO, D, C>(const chunk_args &, hipStream_t); \
  template hipError_t launch_r1_scan<IO, D, C>(const chunk_args &, hipStream_t);

GDN2_INST_R1(float, 16, 16)
GDN2_INST_R1(float, 32, 16)
GDN2_INST_R1(float, 64, 16)
GDN2_INST_R1(float, 128, 16)
GDN2_INST_R1(float, 16, 64)
GDN2_INST_R1(float, 32, 64)
GDN2_INST_R1(float, 64, 64)
GDN2_INST_R1(bf16_t, 16, 16)
GDN2_INST_R1(bf16_t, 32, 16)
GDN2_INST_R1(bf16_t, 64, 16)
GDN2_INST_R1(bf16_t, 128, 16)
GDN2_INST_R1(bf16_t, 16, 64)
GDN2_INST_R1(bf16_t, 32, 64)
GDN2_INST_R1(bf16_t, 64, 64)
GDN2_INST_R1(bf16_t, 128, 64)

}  // namespace gdn2
