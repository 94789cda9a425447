// gdn2_chunk.hip -- chunkwise-parallel GDN-2 forward for gfx950.
//
// The recurrence (see gdn2_recurrent.hip) is re-parallelised over chunks of C
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
// W, Ut, Q', O_intra, Kbar and gamma_C depend only on the chunk's own inputs
// (kernel 1, fully parallel over chunks and heads); the entering state only
// enters through three state-sized products per chunk (kernel 2, sequential
// over chunks, parallel over sequences, heads and 16-column slices of dv).
//
// Numerics of the decay factorisation: every factor exp(g_t - g_s) with s <= t
// is at most 1, but splitting it as gamma_t / gamma_s can overflow.  A and P
// are therefore built per 16-token sub-block with the reference point at the
// start of the row's own sub-block I:
//   A[t][s] = sum_c (b k_t e^{g_t - rho_I}) (e^{rho_I - rho_J}) (k_s e^{rho_J - g_s})
// for s in sub-block J <= I, rho_J = g just before sub-block J.  The first and
// middle factors are <= 1; the last is bounded by the decay over one 16-token
// sub-block.  E, Qchk and Kbar use the chunk start / chunk end and are <= 1.
//
// Matrix products use the fragment convention of gdn2_device.hpp.  Kernel 1
// runs one wave per 16-token sub-block (4 waves for C = 64):
//   phase 1  loads, log2(alpha), in-wave prefix sum over tokens, block totals
//   phase 2  A and P sub-block rows (matrix cores)
//   phase 3  T = (I + A)^{-1}: 16x16 diagonal inverses by forward substitution
//            (every lane solves one column), off-diagonal blocks level by
//            level with T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ (matrix cores)
//   phase 4  W = T E, Ut = T U
//   phase 5  Q' = Qchk - P W (computed transposed, so that it lands in the
//            operand layout kernel 2 reads), O_intra = P Ut
// Intermediates go to the workspace in fragment order, so kernel 2 reads every
// operand with one coalesced 8- or 16-byte load per lane and keeps the state
// in matrix-core accumulators for the whole sequence.
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
  __device__ __forceinline__ f32x4 f() const { return x; }
};
template <> struct raw4<bf16_t> {
  uint2 x;
  __device__ static __forceinline__ raw4 ld(const bf16_t *p) {
    raw4 r;
    r.x = *reinterpret_cast<const uint2 *>(p);
    return r;
  }
  __device__ static __forceinline__ raw4 fill(float v) {
    const uint32_t h = f2bf(v);
    raw4 r;
    r.x.x = h | (h << 16);
    r.x.y = r.x.x;
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

// Per (chunk slot, head) block of intermediates, all tiles fragment-ordered.
// The first SHARED bytes (-W, Q', Kbar^T, gamma_C) are what every column
// slice of the state scan needs; they are copied to LDS as one block.  A
// operands of the scan are stored with their 16-wide k tiles paired
// (tile_off), so one 16-byte load yields a 16x16x32 operand.
template <typename IO, int D, int C> struct blk_layout {
  static constexpr int NB = C / 16, NK = D / 16;
  static constexpr size_t TB = frag<IO>::TILE_BYTES;
  static constexpr size_t WN = 0;                   // rows tt, k tiles over dk: RowFrag(-W)
  static constexpr size_t QP = WN + NB * NK * TB;   // rows tt, k tiles over dk: RowFrag(Q')
  static constexpr size_t KB = QP + NB * NK * TB;   // rows dk tile, k tiles over tokens: RowFrag(Kbar^T)
  static constexpr size_t GAM = KB + NK * NB * TB;  // [D] float gamma_C
  static constexpr size_t SHARED = (GAM + D * sizeof(float) + 1023) & ~static_cast<size_t>(1023);
  static constexpr size_t UT = SHARED;              // [NB][NK] ColFrag(Ut)
  static constexpr size_t OI = UT + NB * NK * TB;   // [NB][NK] ColFrag(O_intra)
  static constexpr size_t BYTES = align256(OI + NB * NK * TB);
};

template <typename IO, int D, int C> size_t chunk_block_bytes() { return blk_layout<IO, D, C>::BYTES; }

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

template <typename IO, int D, int C> struct prep_smem {
  static constexpr int NB = C / 16, NK = D / 16;
  static constexpr int NP = NB * (NB - 1) / 2;  // sub-block pairs J < I
  static constexpr int NT = NB * (NB + 1) / 2;  // sub-block pairs J <= I
  static constexpr int NKS = (NP > NB ? NP : NB);
  static constexpr int TB = frag<IO>::TILE_BYTES;
  float tot[NB][D];                  // per-sub-block sum of log2(alpha)
  float f1[NB][D];                   // exp2(rho_I): decay from chunk start to sub-block I
  float f2[NB][D];                   // exp2(g_C - rho_I): decay from sub-block I to chunk end
  float sig[NP > 0 ? NP : 1][D];     // exp2(rho_I - rho_J) <= 1 for the pair (I, J), J < I
  float ad[NB][16][16];              // diagonal blocks of A, row-major
  // RowFrag(Khat_J * sig_IJ) for each pair (I, J), k tiles paired; after the
  // A/P products the same bytes hold RowFrag(Qchk) tiles [NB][NK]
  alignas(16) unsigned char khs[NKS][NK][TB];
  alignas(16) unsigned char ec[NB][NK][TB];  // ColFrag(E_J), one tile per 16 channels
  alignas(16) unsigned char pr[NT][TB];      // RowFrag(P_IJ)
  alignas(16) unsigned char tcol[NT][TB];    // ColFrag(T_IJ)
  alignas(16) unsigned char trow[NT][TB];    // RowFrag(T_IJ)
};

__device__ __forceinline__ constexpr int pair_index(int I, int J) { return I * (I - 1) / 2 + J; }
__device__ __forceinline__ constexpr int tri_index(int I, int J) { return I * (I + 1) / 2 + J; }

// Kernel 1: per-chunk prep + in-chunk WY/UT factor.  grid: num_slots * H,
// block: 64 * C/16 threads.  Wave I owns the 16-token sub-block I for the
// row-wise phases (loads, decay prefix sums, A and P rows, T rows) and
// column tiles [I*CTW, I*CTW + CTW) of dk and dv for the column-wise phases
// (W, Ut, Q', O_intra), so every wave does the same amount of matrix work.
template <typename IO, int D, int C>
__global__ void __launch_bounds__(64 * (C / 16)) gdn2_chunk_prep_kernel(chunk_args a) {
  constexpr int NB = C / 16, NK = D / 16;
  constexpr int CTW = (NK >= NB) ? NK / NB : 1;  // column tiles per wave
  typedef frag<IO> F;
  typedef frag2<IO> F2;
  typedef blk_layout<IO, D, C> L;
  typedef prep_smem<IO, D, C> SM;
  __shared__ SM sm;

  const int h = blockIdx.x % a.H;
  const int slot = blockIdx.x / a.H;
  int seq, len;
  long t0;
  if (!locate_chunk<C>(slot, a, seq, t0, len))
    return;  // whole workgroup leaves together
  (void)seq;
  const int tid = threadIdx.x;
  const int I = tid >> 6;  // sub-block (row phases) of this wave
  const int lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int t = 16 * I + m;  // token within the chunk
  const bool valid = t < len;
  const int ct0 = I * CTW;    // first column tile (column phases)
  const bool owner = ct0 < NK;
  unsigned char *blk = reinterpret_cast<unsigned char *>(a.blocks) +
                       (static_cast<size_t>(slot) * a.H + h) * a.blk_bytes;
  auto row_of = [&](int tok) { return static_cast<size_t>(t0 + tok) * a.H + h; };
  const IO *qp = static_cast<const IO *>(a.q) + row_of(valid ? t : 0) * D;
  const IO *kp = static_cast<const IO *>(a.k) + row_of(valid ? t : 0) * D;
  const IO *ap = static_cast<const IO *>(a.al) + row_of(valid ? t : 0) * D;
  const IO *bp = static_cast<const IO *>(a.b) + row_of(valid ? t : 0) * D;

  // ---------------- phase 1: loads, log-decay prefix sums, block totals
  raw4<IO> rq[NK], rk[NK], rb[NK];
  f32x4 gl[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const int c0 = 16 * kk + 4 * g;
    if (valid) {
      rq[kk] = raw4<IO>::ld(qp + c0);
      rk[kk] = raw4<IO>::ld(kp + c0);
      rb[kk] = raw4<IO>::ld(bp + c0);
      const f32x4 al = raw4<IO>::ld(ap + c0).f();
#pragma unroll
      for (int i = 0; i < 4; ++i)
        gl[kk][i] = fast_log2(al[i]);
    } else {
      rq[kk] = rk[kk] = rb[kk] = raw4<IO>::fill(0.f);
      gl[kk] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  // values and write gates of every sub-block, for this wave's column tiles
  raw4<IO> rv[NB][CTW], rw[NB][CTW];
#pragma unroll
  for (int J = 0; J < NB; ++J) {
    const int tj = 16 * J + m;
    const bool vj = owner && tj < len;
    const IO *vp = static_cast<const IO *>(a.v) + row_of(vj ? tj : 0) * D;
    const IO *wp = static_cast<const IO *>(a.w) + row_of(vj ? tj : 0) * D;
#pragma unroll
    for (int j = 0; j < CTW; ++j) {
      const int c0 = 16 * (ct0 + j) + 4 * g;
      if (vj) {
        rv[J][j] = raw4<IO>::ld(vp + c0);
        rw[J][j] = raw4<IO>::ld(wp + c0);
      } else {
        rv[J][j] = rw[J][j] = raw4<IO>::fill(0.f);
      }
    }
  }
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      gl[kk][i] = row16_inclusive_scan(gl[kk][i]);
  if (m == 15) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      *reinterpret_cast<f32x4 *>(&sm.tot[I][16 * kk + 4 * g]) = gl[kk];
  }
  __syncthreads();

  // per-channel decay factors between sub-block boundaries
  for (int idx = tid; idx < NB * D; idx += 64 * NB) {
    const int J = idx / D, c = idx - J * D;
    float rho = 0.f, suf = 0.f;
#pragma unroll
    for (int K = 0; K < NB; ++K) {
      const float x = sm.tot[K][c];
      if (K < J)
        rho += x;
      else
        suf += x;
    }
    sm.f1[J][c] = fast_exp2(rho);
    sm.f2[J][c] = fast_exp2(suf);
    float part = 0.f;  // sum of tot over sub-blocks J .. I2-1
#pragma unroll
    for (int I2 = 1; I2 < NB; ++I2) {
      if (I2 > J) {
        part += sm.tot[I2 - 1][c];
        sm.sig[pair_index(I2, J)][c] = fast_exp2(part);
      }
    }
    if (J == 0)
      reinterpret_cast<float *>(blk + L::GAM)[c] = fast_exp2(suf);
  }
  __syncthreads();

  // ---------------- phase 1b: decayed, gated operands
  const F eye = identity_colfrag<IO>(lane);
  F ef[NK], qf[NK], khf[NK], qcf[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const int c0 = 16 * kk + 4 * g;
    const f32x4 f1v = *reinterpret_cast<const f32x4 *>(&sm.f1[I][c0]);
    const f32x4 f2v = *reinterpret_cast<const f32x4 *>(&sm.f2[I][c0]);
    f32x4 f, fi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = fast_exp2(gl[kk][i]);    // e^{g_t - rho_I} <= 1
      fi[i] = fast_exp2(-gl[kk][i]);  // e^{rho_I - g_t} >= 1
    }
    const f32x4 kf = rk[kk].f();
    const f32x4 er = rb[kk].f() * kf * f;
    const f32x4 qr = rq[kk].f() * f;
    const f32x4 kh = kf * fi;
    ef[kk] = F::from(er);
    qf[kk] = F::from(qr);
    khf[kk] = F::from(kh);
    qcf[kk] = F::from(qr * f1v);
    // keys of this sub-block rescaled to the reference point of each later one
#pragma unroll
    for (int I2 = 1; I2 < NB; ++I2) {
      if (I2 > I) {
        const f32x4 s = *reinterpret_cast<const f32x4 *>(&sm.sig[pair_index(I2, I)][c0]);
        F::from(kh * s).st(&sm.khs[pair_index(I2, I)][0][0] + tile_off<IO, NK>(0, kk, lane), 0);
      }
    }
    F::from(transpose_frag(F::from(er * f1v), eye)).st(sm.ec[I][kk], lane);
    F::from(transpose_frag(F::from(kh * f2v), eye)).st(blk + L::KB + tile_off<IO, NB>(kk, I, lane), 0);
  }
  // ColFrag(U_J) = ColFrag(w (.) v) of the own column tiles
  F ucol[NB][CTW];
#pragma unroll
  for (int J = 0; J < NB; ++J)
#pragma unroll
    for (int j = 0; j < CTW; ++j)
      ucol[J][j] = F::from(transpose_frag(F::from(rw[J][j].f() * rv[J][j].f()), eye));
  __syncthreads();

  // ---------------- phase 2: A and P rows of sub-block I, as RowFrag
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
          mma32(accA[J], a2, F2::make(ef[2 * kp], ef[2 * kp + 1]));
          mma32(accP[J], a2, F2::make(qf[2 * kp], qf[2 * kp + 1]));
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const F a1 = F::ld(kb + tile_off<IO, NK>(0, kk, 0), lane);
          mma16(accA[J], a1, ef[kk]);
          mma16(accP[J], a1, qf[kk]);
        }
      }
    } else if (J == I) {
      if constexpr (NK % 2 == 0) {
#pragma unroll
        for (int kp = 0; kp < NK / 2; ++kp) {
          const F2 a2 = F2::make(khf[2 * kp], khf[2 * kp + 1]);
          mma32(accA[J], a2, F2::make(ef[2 * kp], ef[2 * kp + 1]));
          mma32(accP[J], a2, F2::make(qf[2 * kp], qf[2 * kp + 1]));
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          mma16(accA[J], khf[kk], ef[kk]);
          mma16(accP[J], khf[kk], qf[kk]);
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
    if (J <= I)
      F::from(accP[J]).st(sm.pr[tri_index(I, J)], lane);
  }
  F af[NB];
#pragma unroll
  for (int K = 0; K < NB; ++K)
    af[K] = F::from(accA[K]);
  __syncthreads();
  // the rescaled keys are consumed: their bytes now hold RowFrag(Qchk)
  unsigned char *qc_tiles = &sm.khs[0][0][0];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
    qcf[kk].st(qc_tiles + (I * NK + kk) * SM::TB, lane);

  // ---------------- phase 3: T = (I + A)^{-1}
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
  const F trow_ii = F::ld(sm.trow[tri_index(I, I)], lane);
#pragma unroll
  for (int l = 1; l < NB; ++l) {
    if (I >= l) {
      const int J = I - l;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int K = 0; K < NB; ++K)
        if (K >= J && K < I)
          mma16(acc, af[K], F::ld(sm.tcol[tri_index(K, J)], lane));
      f32x4 tij = {0.f, 0.f, 0.f, 0.f};
      mma16(tij, trow_ii, F::from(acc));
      const F tf = F::from(-tij);
      tf.st(sm.tcol[tri_index(I, J)], lane);
      F::from(transpose_frag(tf, eye)).st(sm.trow[tri_index(I, J)], lane);
    }
    __syncthreads();
  }

  // ---------------- phases 4-5, by column tile: W = T E, Ut = T U,
  // Q' = Qchk - P W (computed as Q'^T so it lands as RowFrag), O_intra = P Ut
  if (owner) {
#pragma unroll
    for (int j = 0; j < CTW; ++j) {
      const int ct = ct0 + j;
      F wc[NB], uc[NB];
#pragma unroll
      for (int I2 = 0; I2 < NB; ++I2) {
        f32x4 w = {0.f, 0.f, 0.f, 0.f}, u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = 0; J <= I2; ++J) {
          const F tr = F::ld(sm.trow[tri_index(I2, J)], lane);
          mma16(w, tr, F::ld(sm.ec[J][ct], lane));
          mma16(u, tr, ucol[J][j]);
        }
        wc[I2] = F::from(w);
        uc[I2] = F::from(u);
        uc[I2].st(blk + L::UT + (I2 * NK + ct) * L::TB, lane);
        F::from(transpose_frag(wc[I2], eye)).neg().st(blk + L::WN + tile_off<IO, NK>(I2, ct, lane), 0);
      }
#pragma unroll
      for (int I2 = 0; I2 < NB; ++I2) {
        f32x4 q = F::ld(qc_tiles + (I2 * NK + ct) * SM::TB, lane).to_f32();
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = 0; J <= I2; ++J) {
          const F p = F::ld(sm.pr[tri_index(I2, J)], lane);
          mma16(q, wc[J], p.neg());
          mma16(o, p, uc[J]);
        }
        F::from(q).st(blk + L::QP + tile_off<IO, NK>(I2, ct, lane), 0);
        F::from(o).st(blk + L::OI + (I2 * NK + ct) * L::TB, lane);
      }
    }
  }
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Kernel 2: sequential state scan + output.  A workgroup of NW waves owns one
// (sequence, head) and NW 16-column slices of dv; wave w keeps its slice of
// the state S (dk x 16, float32) in matrix-core accumulators for the whole
// sequence.  Per chunk, the shared -W, Q', Kbar^T, gamma_C block (49 KB for
// bf16, d = 128, C = 64) is copied HBM -> LDS with global_load_lds (no
// register staging) one chunk ahead, into the other of NBUF buffers, while
// the waves compute the current chunk:
//   Z = Ut - W S,  O = O_intra + Q' S  (written to o),  S <- Diag(gamma_C) S + Kbar^T Z.
// Grid: units_pad * (D/16/NW) workgroups, units_pad = N*H rounded up to 8;
// consecutive ids go to the 8 XCDs round-robin and all column groups of one
// head share an XCD (and its L2).
template <typename IO, int D, int C, int NW, int NBUF>
__global__ void __launch_bounds__(64 * NW) gdn2_chunk_scan_kernel(chunk_args a) {
  constexpr int NB = C / 16, NK = D / 16, NG = NK / NW;
  typedef frag<IO> F;
  typedef frag2<IO> F2;
  typedef blk_layout<IO, D, C> L;
  constexpr int NDMA = static_cast<int>(L::SHARED / 1024);  // 1 KB per wave instruction
  __shared__ __attribute__((aligned(16))) unsigned char sbuf[NBUF][L::SHARED];

  const int x = blockIdx.x;
  const int xcd = x & 7, s8 = x >> 3;
  const int unit = (s8 / NG) * 8 + xcd;
  const int cg = s8 % NG;
  if (unit >= a.num_seqs * a.H)
    return;
  const int n = unit / a.H, h = unit - n * a.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  const int vt = cg * NW + wave;
  int c_begin, nchunks;
  long tstart, tend;
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
  const unsigned char *blocks = reinterpret_cast<const unsigned char *>(a.blocks);
  auto blk_of = [&](int c) { return blocks + (static_cast<size_t>(c_begin + c) * a.H + h) * a.blk_bytes; };
  auto dma = [&](int c, int buf) {
    const unsigned char *src = blk_of(c);
    for (int i = wave; i < NDMA; i += NW)
      __builtin_amdgcn_global_load_lds(src + i * 1024 + lane * 16,
                                       (lds_void_t *)(&sbuf[buf][i * 1024]), 16, 0, 0);
  };

  const int col = 16 * vt + m;
  f32x4 S[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[kk][i] = a.S0 ? a.S0[(static_cast<size_t>(unit) * D + 16 * kk + 4 * g + i) * D + col] : 0.f;
  IO *out = static_cast<IO *>(a.o);

  F ut[NB], oi[NB];
  if (nchunks > 0) {
    dma(0, 0);
    const unsigned char *blk = blk_of(0);
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
      ut[tt] = F::ld(blk + L::UT + (tt * NK + vt) * L::TB, lane);
      oi[tt] = F::ld(blk + L::OI + (tt * NK + vt) * L::TB, lane);
    }
  }
  for (int c = 0; c < nchunks; ++c) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // chunk c's block is in sbuf[c % NBUF]; nobody still reads the other buffer
    F utc[NB], oic[NB];
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
      utc[tt] = ut[tt];
      oic[tt] = oi[tt];
    }
    if (NBUF > 1 && c + 1 < nchunks) {
      dma(c + 1, (c + 1) % NBUF);
      const unsigned char *blk = blk_of(c + 1);
#pragma unroll
      for (int tt = 0; tt < NB; ++tt) {
        ut[tt] = F::ld(blk + L::UT + (tt * NK + vt) * L::TB, lane);
        oi[tt] = F::ld(blk + L::OI + (tt * NK + vt) * L::TB, lane);
      }
    }
    const unsigned char *sb = sbuf[c % NBUF];
    const long t0 = tstart + static_cast<long>(c) * C;
    const int len = (tend - t0) < C ? static_cast<int>(tend - t0) : C;

    F sf[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      sf[kk] = F::from(S[kk]);
    F zf[NB];
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
      f32x4 z = utc[tt].to_f32();
      f32x4 o = oic[tt].to_f32();
      if constexpr (NK % 2 == 0) {
#pragma unroll
        for (int k2 = 0; k2 < NK / 2; ++k2) {
          const F2 sb2 = F2::make(sf[2 * k2], sf[2 * k2 + 1]);
          mma32(z, F2::ld(sb + L::WN + tile_off<IO, NK>(tt, 2 * k2, 0), lane), sb2);
          mma32(o, F2::ld(sb + L::QP + tile_off<IO, NK>(tt, 2 * k2, 0), lane), sb2);
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          mma16(z, F::ld(sb + L::WN + tile_off<IO, NK>(tt, kk, 0), lane), sf[kk]);
          mma16(o, F::ld(sb + L::QP + tile_off<IO, NK>(tt, kk, 0), lane), sf[kk]);
        }
      }
      zf[tt] = F::from(z);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * tt + 4 * g + i;
        if (t < len)
          out[(static_cast<size_t>(t0 + t) * a.H + h) * D + col] = io<IO>::from_f(o[i]);
      }
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const f32x4 gam = *reinterpret_cast<const f32x4 *>(sb + L::GAM + (16 * kk + 4 * g) * sizeof(float));
      S[kk] *= gam;
      if constexpr (NB % 2 == 0) {
#pragma unroll
        for (int t2 = 0; t2 < NB / 2; ++t2)
          mma32(S[kk], F2::ld(sb + L::KB + tile_off<IO, NB>(kk, 2 * t2, 0), lane),
                F2::make(zf[2 * t2], zf[2 * t2 + 1]));
      } else {
#pragma unroll
        for (int tt = 0; tt < NB; ++tt)
          mma16(S[kk], F::ld(sb + L::KB + tile_off<IO, NB>(kk, tt, 0), lane), zf[tt]);
      }
    }
    if (NBUF == 1 && c + 1 < nchunks) {
      __syncthreads();  // everyone is done with the only buffer
      dma(c + 1, 0);
      const unsigned char *blk = blk_of(c + 1);
#pragma unroll
      for (int tt = 0; tt < NB; ++tt) {
        ut[tt] = F::ld(blk + L::UT + (tt * NK + vt) * L::TB, lane);
        oi[tt] = F::ld(blk + L::OI + (tt * NK + vt) * L::TB, lane);
      }
    }
  }
  if (a.S_final) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a.S_final[(static_cast<size_t>(unit) * D + 16 * kk + 4 * g + i) * D + col] = S[kk][i];
  }
}

// Kernel 0: per-sequence chunk offsets for packed input (integer only).
// One workgroup of 256 threads; offsets[n] = sum_{m<n} ceil(len_m / C).
__global__ void __launch_bounds__(256)
    gdn2_chunk_table_kernel(const int32_t *__restrict__ cu, int N, int C, int32_t *offsets) {
  __shared__ int part[256];
  const int tid = threadIdx.x;
  const int per = (N + 255) / 256;
  const int beg = tid * per;
  const int end = (beg + per < N) ? beg + per : N;
  int s = 0;
  for (int n = beg; n < end; ++n)
    s += (cu[n + 1] - cu[n] + C - 1) / C;
  part[tid] = s;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < 256; ++i) {
      const int vv = part[i];
      part[i] = acc;
      acc += vv;
    }
    offsets[N] = acc;
  }
  __syncthreads();
  int acc = part[tid];
  for (int n = beg; n < end; ++n) {
    offsets[n] = acc;
    acc += (cu[n + 1] - cu[n] + C - 1) / C;
  }
}

// ------------------------------------------------------------- launchers --
template <typename IO, int D, int C> hipError_t launch_chunk_prep(const chunk_args &a, hipStream_t st) {
  if (a.num_slots > 0)
    hipLaunchKernelGGL((gdn2_chunk_prep_kernel<IO, D, C>), dim3(a.num_slots * a.H), dim3(64 * (C / 16)),
                       0, st, a);
  return hipGetLastError();
}

template <typename IO, int D, int C, int NW>
hipError_t launch_scan_nw(const chunk_args &a, hipStream_t st) {
  typedef blk_layout<IO, D, C> L;
  constexpr int NBUF = (2 * L::SHARED <= 150 * 1024) ? 2 : 1;
  const int units = a.num_seqs * a.H;
  const int units_pad = (units + 7) / 8 * 8;
  hipLaunchKernelGGL((gdn2_chunk_scan_kernel<IO, D, C, NW, NBUF>), dim3(units_pad * (D / 16 / NW)),
                     dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

// Workgroups share the per-chunk block in LDS across NW = 4 waves when that
// still gives at least one workgroup per compute unit; with few (sequence,
// head) units (long sequences, small batch) every wave gets its own
// workgroup so that all of them can run.
template <typename IO, int D, int C> hipError_t launch_chunk_scan(const chunk_args &a, hipStream_t st) {
  constexpr int NK = D / 16;
  const long wgs4 = static_cast<long>(a.num_seqs) * a.H * NK / 4;
  if constexpr (NK >= 4) {
    if (wgs4 >= 256)
      return launch_scan_nw<IO, D, C, 4>(a, st);
  }
  return launch_scan_nw<IO, D, C, 1>(a, st);
}

hipError_t launch_chunk_table(const int32_t *cu, int N, int C, int32_t *offsets, hipStream_t st) {
  hipLaunchKernelGGL(gdn2_chunk_table_kernel, dim3(1), dim3(256), 0, st, cu, N, C, offsets);
  return hipGetLastError();
}

#define GDN2_INST_CHUNK(IO, D, C)                                                           \
  template size_t chunk_block_bytes<IO, D, C>();                                            \
  template hipError_t launch_chunk_prep<IO, D, C>(const chunk_args &, hipStream_t);         \
  template hipError_t launch_chunk_scan<IO, D, C>(const chunk_args &, hipStream_t);

GDN2_INST_CHUNK(float, 16, 16)
GDN2_INST_CHUNK(float, 32, 16)
GDN2_INST_CHUNK(float, 64, 16)
GDN2_INST_CHUNK(float, 128, 16)
GDN2_INST_CHUNK(float, 16, 64)
GDN2_INST_CHUNK(float, 32, 64)
GDN2_INST_CHUNK(float, 64, 64)
GDN2_INST_CHUNK(float, 128, 64)
GDN2_INST_CHUNK(bf16_t, 16, 16)
GDN2_INST_CHUNK(bf16_t, 32, 16)
GDN2_INST_CHUNK(bf16_t, 64, 16)
GDN2_INST_CHUNK(bf16_t, 128, 16)
GDN2_INST_CHUNK(bf16_t, 16, 64)
GDN2_INST_CHUNK(bf16_t, 32, 64)
GDN2_INST_CHUNK(bf16_t, 64, 64)
GDN2_INST_CHUNK(bf16_t, 128, 64)

}  // namespace gdn2
