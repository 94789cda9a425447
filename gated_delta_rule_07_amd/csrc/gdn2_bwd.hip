// gdn2_bwd.hip -- chunked backward of the GDN-2 recurrence (gfx950).
//
// The pages ask for gradients through both gates, taken inside the chunked
// products (aiexpert.news/pt, method paragraph; aixai.ru blog, section on how
// the method is implemented in practice).  Given dL/do and dL/dS_final, the
// backward runs, after the forward's per-chunk prep:
//   1. the state scan in states mode: the state S entering every chunk;
//   2. gdn2_bwd_dstate_kernel: the reverse scan of dH, the gradient of the
//      state leaving each chunk.  With the chunk form of the forward
//        Z = Ut - W S,  O = O_intra + Q' S,  S_C = Diag(gamma) S + Kbar^T Z,
//      the gradient entering the chunk is
//        dS = Diag(gamma) dH + Q'^T dO - W^T (Kbar dH),
//      and the one entering the first chunk is dL/dS0;
//   3. gdn2_bwd_grad_kernel: every chunk in parallel, given S and dH,
//      differentiates the chunk's own products (below) down to dq, dk, dv,
//      dalpha, db, dw.
//
// Chunk form differentiated by the gradient kernel (one chunk of C tokens,
// one head; g_t = sum of ln alpha over the chunk's tokens up to t, per key
// channel; rho_I = g before 16-token sub-block I; e = b (.) k; u = w (.) v):
//   QS = q e^{g}, ES = e e^{g}, KB = k e^{g_C - g}        (chunk-start scale)
//   QR = q e^{g - rho_I(t)}, ER = e e^{g - rho_I(t)}       (own sub-block)
//   K~ = k e^{rho_{J+1} - g}  (key s of sub-block J, to the end of J)
//   A = strict-lower(ER X K~^T), P = lower(QR X K~^T) with X the factor
//       e^{rho_I - rho_{J+1}} between the pair's sub-blocks: every factor
//       e^{g_t - g_s} is a product of bounded ones.  Each factor is a sum of
//       log decays taken directly (never the difference of two prefix
//       sums), so alpha = 0 (ln = -inf) gives exact zeros, not NaN.  A
//       diagonal pair (I = J) takes X = e^{-(sub-block's log decay)}, bounded
//       while that decay is above e^-DIAG_LIM_LN; a chunk with a stronger one
//       (or alpha = 0) is left to the kernel's PW variant, which forms the
//       diagonal blocks and their gradients pair by pair with running
//       products of the alphas
//   T = (I + A)^{-1},  Y = U - ES S,  Z = T Y
//   O = QS S + P Z,  S_C = Diag(e^{g_C}) S + KB^T Z.
// Reverse mode: dZ = P^T dO + KB dH, dY = T^T dZ, dA = -strict-lower(dY Z^T),
// dP = lower(dO Z^T), dQS = dO S^T, dES = -dY S^T, dKB = Z dH^T,
// dQR_I = dP_I KR_I, dER_I = dA_I KR_I, dKR_I = dP_I^T QR_I + dA_I^T ER_I,
// dgamma = rowsum(dH (.) S).  Each scaled copy X = x e^{phi} gives
// dx += dX e^{phi} and dphi = x (.) dx-contribution; phi is +g_t, g_t - rho,
// rho - g_s or g_C - g_s (the rho cancel and are held constant).  Finally
// d ln(alpha_s) = sum over t >= s of dg_t (g_C counts as the chunk's last
// row), dalpha = d ln(alpha) / alpha, dv = dY (.) w, dw = dY (.) v,
// db = k (.) de, dk += b (.) de.
#include "gdn2_kernels.hpp"
#include "gdn2_wy.hpp"

#include <type_traits>

namespace gdn2 {

// ------------------------------------------------------- reverse dH scan --
// NSPL workgroups per (sequence, head), placed on one XCD (their common tile
// reads hit its L2), each with one wave per 16-column slice of dH of its
// share (dk x 16 float32 in matrix-core accumulators): with two, a batch of
// 128 (sequence, head) units fills the 256 compute units.  Per chunk, from the last:
// the waves re-lay the chunk's Kbar, Q'^T and -W^T tiles (stored by the prep
// as RowFrag(Kbar^T), RowFrag(Q'), RowFrag(-W)) into LDS with one identity
// product each, then every wave stores its slice of dH (the gradient of the
// state leaving the chunk, as state_tiles fragments) and updates it.
template <int D> struct dstate_cfg {
  static constexpr int NK = D / 16;
  static constexpr int NSPL = NK >= 2 ? 2 : 1;  // workgroups per (sequence, head)
  static constexpr int NW = NK / NSPL;          // waves (dv tiles) per workgroup
};

template <typename IO, int D, int C>
__global__ void __launch_bounds__(64 * dstate_cfg<D>::NW) gdn2_bwd_dstate_kernel(bwd_args ba) {
  const chunk_args &a = ba.f;
  constexpr int NB = C / 16, NK = D / 16, NSPL = dstate_cfg<D>::NSPL, NW = dstate_cfg<D>::NW, NT = NB * NK;
  static_assert(64 * NW >= D, "gamma_C is loaded one channel per thread");
  typedef frag<IO> F;
  typedef blk_layout<IO, D, C> L;
  constexpr size_t TB = F::TILE_BYTES;
  // [0, NT): RowFrag(Kbar) tiles (tt, kk); [NT, 2NT): RowFrag(Q'^T) tiles
  // (kk, tt); [2NT, 3NT): RowFrag(-W^T) tiles (kk, tt); then gamma_C
  __shared__ __attribute__((aligned(16))) unsigned char sm[3 * NT * TB + D * sizeof(float)];
  float *gam = reinterpret_cast<float *>(sm + 3 * NT * TB);

  const int x = static_cast<int>(blockIdx.x), xcd = x & 7, s8 = x >> 3;
  const int unit = (s8 / NSPL) * 8 + xcd, grp = s8 % NSPL;
  if (unit >= a.num_seqs * a.H)
    return;  // the whole workgroup
  const int n = unit / a.H, h = unit - n * a.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  const int j = grp * NW + wave;  // dv tile of this wave
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
  f32x4 dh[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dh[kk][i] = ba.dSf ? ba.dSf[(static_cast<size_t>(unit) * D + 16 * kk + 4 * g + i) * D + 16 * j + m] : 0.f;
  const F eye = identity_colfrag<IO>(lane);
  const IO *dout = static_cast<const IO *>(ba.dout);

  // software pipeline: chunk c - 1's operand tiles, gamma and dO are loaded
  // into registers while chunk c is computed, and laid into LDS after it
  constexpr int PPW = (3 * NT + NW - 1) / NW;  // tiles per wave
  F raw[PPW], dof[NB];
  IO dor[NB][4];  // raw dO elements of the next chunk (rows past its end: masked at commit)
  int lenn = 0;
  float gamv = 0.f;
  auto issue = [&](int c) {
    const size_t slot = static_cast<size_t>(c_begin + c);
    const unsigned char *blk = reinterpret_cast<const unsigned char *>(a.blocks) + (slot * a.H + h) * a.blk_bytes;
    const long t0 = tstart + static_cast<long>(c) * C;
    const int len = (tend - t0) < C ? static_cast<int>(tend - t0) : C;
#pragma unroll
    for (int r = 0; r < PPW; ++r) {
      const int p = wave + r * NW;
      if (p < 3 * NT) {
        const int which = p / NT, q2 = p - which * NT;
        if (which == 0) {
          const int tt = q2 / NK, kk = q2 - tt * NK;
          raw[r] = F::ld_at(blk + L::KB + tile_off<IO, NB>(kk, tt, lane));
        } else {
          const int kk = q2 / NB, tt = q2 - kk * NB;
          raw[r] = F::ld_at(blk + (which == 1 ? L::QP : L::WN) + tile_off<IO, NK>(tt, kk, lane));
        }
      }
    }
    if (threadIdx.x < D)
      gamv = reinterpret_cast<const float *>(blk + L::GAM)[threadIdx.x];
    // ColFrag(dO tile (tt, j)): rows 16 tt + 4 g + i, column 16 j + m.
    // Rows past the end read the chunk's first row (every load unconditional,
    // so none waits for another); they are zeroed at commit.
    lenn = len;
    const IO *dbase = dout + (static_cast<size_t>(t0) * a.H + h) * D + 16 * j;  // uniform
#pragma unroll
    for (int tt = 0; tt < NB; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 16 * tt + 4 * g + i;
        const unsigned off = static_cast<unsigned>((t < len ? t : 0) * a.H * D + m);
        dor[tt][i] = dbase[off];
      }
  };
  auto commit = [&]() {
#pragma unroll
    for (int r = 0; r < PPW; ++r) {
      const int p = wave + r * NW;
      if (p < 3 * NT)
        F::from(transpose_io(raw[r], eye, lane)).st(sm + static_cast<size_t>(p) * TB, lane);
    }
    if (threadIdx.x < D)
      gam[threadIdx.x] = gamv;
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
      f32x4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        x[i] = (16 * tt + 4 * g + i < lenn) ? io<IO>::to_f(dor[tt][i]) : 0.f;
      dof[tt] = F::from(x);
    }
  };
  if (nchunks > 0) {
    issue(nchunks - 1);
    commit();
  }
  lds_barrier();
  for (int c = nchunks - 1; c >= 0; --c) {
    const size_t slot = static_cast<size_t>(c_begin + c);
    issue(c > 0 ? c - 1 : 0);  // on the last step a harmless re-read, so no branch
    typedef state_tiles<IO, D> ST_;
    unsigned char *dp = reinterpret_cast<unsigned char *>(ba.dstates) + (slot * a.H + h) * ST_::BYTES;
    F dhf[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      dhf[kk] = F::from(dh[kk]);  // ColFrag(dH tile (kk, j))
      dhf[kk].st(dp + ST_::COL + ST_::off(kk, j), lane);
      if constexpr (ST_::HAS_ROW)
        F::from(transpose_io(dhf[kk], eye, lane)).st(dp + ST_::ROW + ST_::off(kk, j), lane);
    }
    F xf[NB];  // Kbar dH, ColFrag tiles (tt, j)
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        mm_io(x, F::ld(sm + static_cast<size_t>(tt * NK + kk) * TB, lane), dhf[kk]);
      xf[tt] = F::from(x);
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const f32x4 gm = *reinterpret_cast<const f32x4 *>(gam + 16 * kk + 4 * g);
      dh[kk] *= gm;
#pragma unroll
      for (int tt = 0; tt < NB; ++tt) {
        mm_io(dh[kk], F::ld(sm + static_cast<size_t>(NT + kk * NB + tt) * TB, lane), dof[tt]);
        mm_io(dh[kk], F::ld(sm + static_cast<size_t>(2 * NT + kk * NB + tt) * TB, lane), xf[tt]);
      }
    }
    lds_barrier();  // LDS of chunk c is no longer read
    if (c > 0)
      commit();
    lds_barrier();  // chunk c - 1 is in LDS
  }
  if (ba.dS0) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ba.dS0[(static_cast<size_t>(unit) * D + 16 * kk + 4 * g + i) * D + 16 * j + m] = dh[kk][i];
  }
}

// --------------------------------------------------- per-chunk gradients --
// LDS of one gradient workgroup, byte offsets.  Row-major matrices with
// padded pitches:
//   KT  : the scaled keys K~ (C x D)
//   YZ  : Y, then Z (C x D)
//   ST  : T (C x C), float32
//   DOZ : A (C x C, float32) until Z is formed, then dO, then dZ (C x D)
//   SP  : P (C x C)
// K~, Y/Z, dO/dZ and P are only ever read as matrix-core operands, so they
// are kept in LT, the operand type (bfloat16 for bfloat16 inputs: the stored
// value is the one the product rounds to), with pitches PDL = D + 4 and
// PCL = C + 4 elements; A and T, which the triangular solve reads, stay
// float32 with pitch PC = C + 4.  Above them: BTOT (the NB sub-blocks' log
// decays), DGAM, one strong-decay flag per sub-block and, in the PW variant,
// DIAG (dA_II and dP_II, 16 x 16 floats each, per sub-block).  Once the
// products are done the bottom of the LDS is reused for the dK~ sums of the
// NB sub-blocks (DKS, NK tiles of 256 floats each) and the per-sub-block sums
// GTOT and KBS.  For bfloat16 the chunk's S and dH tiles are staged at the
// top (STG, below).
template <typename LT, int D, int C, bool PW = false> struct bwd_lds {
  static constexpr int NB = C / 16, NK = D / 16, PC = C + 4, PDL = D + 4, PCL = C + 4;
  static constexpr size_t SZ_CD = sizeof(LT) * C * PDL, SZ_CC = sizeof(float) * C * PC;
  static constexpr size_t KT = 0, YZ = KT + SZ_CD, ST = YZ + SZ_CD, DOZ = ST + SZ_CC,
                          SP = DOZ + (SZ_CD > SZ_CC ? SZ_CD : SZ_CC), BTOT = SP + sizeof(LT) * C * PCL,
                          DGAM = BTOT + sizeof(float) * NB * D, PWF = DGAM + sizeof(float) * D,
                          DIAG = PWF + sizeof(float) * NB, STG = DIAG + (PW ? sizeof(float) * NB * 512 : 0);
  // STAGE: the chunk's entering state S and leaving-state gradient dH are
  // copied into LDS (STG: S then dH, one fragment layout at a time) instead
  // of every wave reading them from global memory
  static constexpr size_t STB = static_cast<size_t>(NK) * NK * frag<LT>::TILE_BYTES;
  static constexpr bool STAGE = sizeof(LT) == 2 && STG + 2 * STB <= 160 * 1024;
  static constexpr size_t BYTES = STG + (STAGE ? 2 * STB : 0);
  static constexpr size_t DKS = 0, GTOT = DKS + sizeof(float) * NB * NK * 256, KBS = GTOT + sizeof(float) * NB * D;
  static_assert(KBS + sizeof(float) * NB * D <= BTOT, "the dK~ and sub-block sums fit below BTOT");
  static_assert(SZ_CD % 16 == 0 && SZ_CC % 16 == 0 && (sizeof(LT) * C * PCL) % 16 == 0, "16-byte aligned regions");
};

// Fragments of a 16 x 16 tile at (r0, c0) of a row-major float32 matrix with
// row pitch `pitch` (LDS or global): RowFrag (lane (m, g) holds row r0 + m,
// columns c0 + 4g .. +3) and ColFrag (lane (c, g) holds rows r0 + 4g .. +3 of
// column c0 + c).
__device__ __forceinline__ f32x4 ld_rowf(const float *M, int pitch, int r0, int c0, int lane) {
  return *reinterpret_cast<const f32x4 *>(M + static_cast<size_t>(r0 + (lane & 15)) * pitch + c0 + 4 * (lane >> 4));
}
__device__ __forceinline__ f32x4 ld_colf(const float *M, int pitch, int r0, int c0, int lane) {
  const float *p = M + static_cast<size_t>(r0 + 4 * (lane >> 4)) * pitch + c0 + (lane & 15);
  f32x4 x;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    x[i] = p[static_cast<size_t>(i) * pitch];
  return x;
}
__device__ __forceinline__ void st_rowf(float *M, int pitch, int r0, int c0, int lane, f32x4 x) {
  *reinterpret_cast<f32x4 *>(M + static_cast<size_t>(r0 + (lane & 15)) * pitch + c0 + 4 * (lane >> 4)) = x;
}
__device__ __forceinline__ void st_colf(float *M, int pitch, int r0, int c0, int lane, f32x4 x) {
  float *p = M + static_cast<size_t>(r0 + 4 * (lane >> 4)) * pitch + c0 + (lane & 15);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    p[static_cast<size_t>(i) * pitch] = x[i];
}

// Keeps the lower triangle of a diagonal tile: ColFrag element (row 4g+i,
// column c) or RowFrag element (row m, column 4g+i); strict drops the diagonal.
__device__ __forceinline__ f32x4 tri_col(f32x4 v, int lane, bool strict) {
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (strict ? (4 * g + i <= c) : (4 * g + i < c))
      v[i] = 0.f;
  return v;
}
__device__ __forceinline__ f32x4 tri_row(f32x4 v, int lane, bool strict) {
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (strict ? (r <= 4 * g + i) : (r < 4 * g + i))
      v[i] = 0.f;
  return v;
}

// The same tiles of a row-major LDS matrix of element type T (pitch in
// elements) as operand fragments of type T, and RowFrag / ColFrag stores
// rounded to T.  For T = bfloat16 a RowFrag is one 8-byte access per lane
// and a ColFrag four 2-byte ones.
template <typename T> __device__ __forceinline__ frag<T> ldm_row(const T *M, int pitch, int r0, int c0, int lane) {
  return frag<T>::ld_at(M + static_cast<size_t>(r0 + (lane & 15)) * pitch + c0 + 4 * (lane >> 4));
}
template <typename T> __device__ __forceinline__ frag<T> ldm_col(const T *M, int pitch, int r0, int c0, int lane) {
  if constexpr (sizeof(T) == 4) {
    return frag<T>::from(ld_colf(M, pitch, r0, c0, lane));
  } else {
    const T *p = M + static_cast<size_t>(r0 + 4 * (lane >> 4)) * pitch + c0 + (lane & 15);
    frag<T> f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.v[i] = static_cast<short>(p[static_cast<size_t>(i) * pitch]);
    return f;
  }
}
template <typename T> __device__ __forceinline__ void stm_row(T *M, int pitch, int r0, int c0, int lane, f32x4 x) {
  frag<T>::from(x).st_at(M + static_cast<size_t>(r0 + (lane & 15)) * pitch + c0 + 4 * (lane >> 4));
}
template <typename T> __device__ __forceinline__ void stm_col(T *M, int pitch, int r0, int c0, int lane, f32x4 x) {
  if constexpr (sizeof(T) == 4) {
    st_colf(M, pitch, r0, c0, lane, x);
  } else {
    const frag<T> f = frag<T>::from(x);
    T *p = M + static_cast<size_t>(r0 + 4 * (lane >> 4)) * pitch + c0 + (lane & 15);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      p[static_cast<size_t>(i) * pitch] = static_cast<T>(f.v[i]);
  }
}

// One workgroup per chunk-head, one wave per 16-token sub-block: wave I keeps
// the rows of sub-block I (q, k, e, g, dO, Z, dY and the gradient
// accumulators) as RowFrag slabs in registers and computes every product
// whose result lives on those rows.  A product X_I M with X_I its own rows is
// taken as M^T X_I^T (operands swapped), which leaves the result in the same
// RowFrag layout.  What other waves need goes through LDS.  Decay factors
// e^{g_t - g_s} are split at rho_J, the cumulative log decay at the end of
// the key's sub-block J: K~_s = k_s e^{rho_J - g_s} <= 1 is stored once per
// row, and the query/erase side of row t takes e^{g_t - rho_J} (<= 1 for
// J < I, bounded by one sub-block's decay for J = I).
// Input modes of the gradient kernel: per-channel inputs, KDA (b and w per
// (token, head)), Gated DeltaNet (also alpha), and any other combination of
// the gate layouts and layer prep read from chunk_args::gates at run time.
enum { BG_PLAIN = 0, BG_KDA = 1, BG_GDN = 2, BG_FLAGS = 3 };

// Decay over a sub-block below e^-DIAG_LIM_LN (= 2^-64) in some channel: the
// chunk goes to the PW variant.
constexpr float DIAG_LIM_LN = 44.3614195558365f;

// PW = false: every chunk whose sub-blocks all decay less than that; it
// records for each chunk-head whether it left it (ba.pwflag).  PW = true:
// launched after it, the chunks it left (every diagonal pair formed pairwise
// from the chunk's inputs); the others exit at once.
template <typename IO, int D, int C, typename CT, int GM, bool PW = false>
__global__ void __launch_bounds__(64 * (C / 16)) gdn2_bwd_grad_kernel(bwd_args ba) {
  constexpr bool GN = GM != BG_PLAIN;
  const chunk_args &a = ba.f;
  static_assert(std::is_same<CT, IO>::value, "LDS operands are kept in the I/O type");
  typedef CT LT;
  typedef bwd_lds<LT, D, C, PW> L;
  constexpr int NB = C / 16, NK = D / 16, PC = L::PC, PDL = L::PDL, PCL = L::PCL;
  __shared__ __attribute__((aligned(16))) unsigned char smb[L::BYTES];
  LT *KT = reinterpret_cast<LT *>(smb + L::KT), *YZ = reinterpret_cast<LT *>(smb + L::YZ);
  LT *DOZ = reinterpret_cast<LT *>(smb + L::DOZ), *sP = reinterpret_cast<LT *>(smb + L::SP);
  float *sT = reinterpret_cast<float *>(smb + L::ST), *sA = reinterpret_cast<float *>(smb + L::DOZ);
  float *btot = reinterpret_cast<float *>(smb + L::BTOT), *gtot = reinterpret_cast<float *>(smb + L::GTOT);
  float *kbs = reinterpret_cast<float *>(smb + L::KBS), *dgam = reinterpret_cast<float *>(smb + L::DGAM);
  float *pwf = reinterpret_cast<float *>(smb + L::PWF), *diag = reinterpret_cast<float *>(smb + L::DIAG);

  const int slot = static_cast<int>(blockIdx.x / a.H), h = static_cast<int>(blockIdx.x - slot * a.H);
  if constexpr (PW) {
    if (!ba.pwflag[blockIdx.x])
      return;  // the whole workgroup: this chunk-head is done
  }
  int seq, len;
  long t0;
  if (!locate_chunk<C>(slot, a, seq, t0, len))
    return;  // the whole workgroup
  (void)seq;
  const int I = threadIdx.x >> 6, lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const int t = 16 * I + m;
  const bool valid = t < len;
  const size_t row = (static_cast<size_t>(t0 + (valid ? t : 0)) * a.H + h) * D;
  typedef frag<IO> F;
  typedef state_tiles<IO, D> ST_;
  // S and dH of this chunk as fragment tiles: ColFrag at ST_::COL, RowFrag at ST_::ROW
  const unsigned char *__restrict__ St =
      reinterpret_cast<const unsigned char *>(a.states) + (static_cast<size_t>(slot) * a.H + h) * ST_::BYTES;
  const unsigned char *__restrict__ Ht =
      reinterpret_cast<const unsigned char *>(ba.dstates) + (static_cast<size_t>(slot) * a.H + h) * ST_::BYTES;
  const IO *__restrict__ q = static_cast<const IO *>(a.q);
  const IO *__restrict__ k = static_cast<const IO *>(a.k);
  const IO *__restrict__ v = static_cast<const IO *>(a.v);
  const IO *__restrict__ al = static_cast<const IO *>(a.al);
  const IO *__restrict__ b = static_cast<const IO *>(a.b);
  const IO *__restrict__ w = static_cast<const IO *>(a.w);
  const IO *__restrict__ dout = static_cast<const IO *>(ba.dout);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // sums of whole sub-blocks' log decays (btot), for this lane's RowFrag
  // columns of tile kk: sub-blocks lo .. hi - 1 (never a difference, so
  // -inf stays -inf)
  auto tot_sum = [&](int lo, int hi, int kk) {
    f32x4 r = zero4;
    for (int J2 = lo; J2 < hi; ++J2)
      r += *reinterpret_cast<const f32x4 *>(btot + J2 * D + 16 * kk + 4 * g);
    return r;
  };
  // cumulative log decay at the end of sub-block J (finite without PW)
  auto rho_end = [&](int J, int kk) { return tot_sum(0, J + 1, kk); };
  auto ex4 = [](f32x4 x) {
    f32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      y[i] = __expf(x[i]);
    return y;
  };
  // Input modes (GN): b, w or alpha given per (token, head) ([B, T, H], one
  // value broadcast over the channels), and layer prep (q, k raw, b and w
  // logits, alpha as the float32 natural-log decay).  Every read of an input
  // goes through these, which give the recurrence's inputs; without GN they
  // are the plain per-channel loads.
  const uint32_t gates = GM == BG_FLAGS ? a.gates
                        : GM == BG_KDA  ? (GATE_SCALAR_B | GATE_SCALAR_W)
                        : GM == BG_GDN  ? (GATE_SCALAR_B | GATE_SCALAR_W | GATE_SCALAR_ALPHA)
                                        : 0u;
  const bool LPm = (gates & GATE_LAYER_PREP) != 0, SBm = (gates & GATE_SCALAR_B) != 0,
             SWm = (gates & GATE_SCALAR_W) != 0, SAm = (gates & GATE_SCALAR_ALPHA) != 0;
  const size_t srow = row / D;  // index of this row in a [B, T, H] input
  const float *__restrict__ lga = static_cast<const float *>(a.al);
  float qs = 1.f, ks = 1.f;  // 1 / |q|, 1 / |k| of this row (layer prep)
  auto sig4 = [](f32x4 x) {
    f32x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      y[i] = 1.f / (1.f + __expf(-x[i]));
    return y;
  };
  auto ld_gate = [&](const IO *p, bool scalar, int c0) -> f32x4 {
    f32x4 x;
    if (GN && scalar) {
      const float e = io<IO>::to_f(p[srow]);
      x = f32x4{e, e, e, e};
    } else {
      x = io<IO>::load4(p + row + c0);
    }
    return (GN && LPm) ? sig4(x) : x;
  };
  auto ld_b = [&](int c0) { return ld_gate(b, SBm, c0); };
  // alpha itself (not under layer prep)
  auto ld_alpha = [&](int c0) -> f32x4 {
    if (GN && SAm) {
      const float e = io<IO>::to_f(al[srow]);
      return f32x4{e, e, e, e};
    }
    return io<IO>::load4(al + row + c0);
  };
  // ln(alpha)
  auto ld_logalpha = [&](int c0) -> f32x4 {
    if (GN && LPm) {
      if (SAm) {
        const float e = lga[srow];
        return f32x4{e, e, e, e};
      }
      return *reinterpret_cast<const f32x4 *>(lga + row + c0);
    }
    f32x4 x = ld_alpha(c0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = __logf(x[i]);
    return x;
  };
  // sum over the row's D channels: this lane's four of tile kk and the three
  // other lanes of the row (lanes m + 16 g)
  auto row_sum = [](float x) {
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    return x;
  };

  // ---- rows of the sub-block; gv = cumulative ln(alpha) within the
  // sub-block (g_t - rho_I); PW: kfac = e^{rho_{I+1} - g_t} (the key's
  // factor, from the suffix sums; otherwise key_fac forms it on use)
  f32x4 qv[NK], kv[NK], ev[NK], gv[NK], kfac[PW ? NK : 1];
  {
    // every row load first, then the arithmetic
    raw4<IO> rq[NK], rk[NK], rb[NK], ra[NK];
    if constexpr (!GN) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const int c0 = 16 * kk + 4 * g;
        rq[kk] = raw4<IO>::ld(q + row + c0);
        rk[kk] = raw4<IO>::ld(k + row + c0);
        rb[kk] = raw4<IO>::ld(b + row + c0);
        ra[kk] = raw4<IO>::ld(al + row + c0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const int c0 = 16 * kk + 4 * g;
        rq[kk] = raw4<IO>::ld(q + row + c0);
        rk[kk] = raw4<IO>::ld(k + row + c0);
      }
      if (LPm) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const f32x4 x = rq[kk].f(), y = rk[kk].f();
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sq += x[i] * x[i];
            sk += y[i] * y[i];
          }
        }
        sq = row_sum(sq);
        sk = row_sum(sk);
        qs = sq > 0.f ? __frsqrt_rn(sq) : 0.f;
        ks = sk > 0.f ? __frsqrt_rn(sk) : 0.f;
      }
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int c0 = 16 * kk + 4 * g;
      f32x4 qq = rq[kk].f() * qs, kq = rk[kk].f() * ks, bq, lq;
      if constexpr (!GN) {
        bq = rb[kk].f();
        lq = ra[kk].f();
#pragma unroll
        for (int i = 0; i < 4; ++i)
          lq[i] = __logf(lq[i]);
      } else {
        bq = ld_b(c0);
        lq = ld_logalpha(c0);
      }
      if (!valid) {
        qq = kq = bq = lq = zero4;
      }
      qv[kk] = qq;
      kv[kk] = kq;
      ev[kk] = bq * kq;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gv[kk][i] = row16_inclusive_scan(lq[i]);  // g_t - rho_I
        if constexpr (PW)
          kfac[PW ? kk : 0][i] = __expf(row16_exclusive_suffix(lq[i]));  // e^{rho_{I+1} - g_t}
      }
    }
  }
  {
    float mn = 0.f;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        mn = fminf(mn, gv[kk][i]);
    const bool pw_wave = __ballot(m == 15 && mn < -DIAG_LIM_LN) != 0;
    if (lane == 0)
      pwf[I] = pw_wave ? 1.f : 0.f;
  }
  if (m == 15) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      *reinterpret_cast<f32x4 *>(btot + I * D + 16 * kk + 4 * g) = gv[kk];
  }
  lds_barrier();
  if constexpr (!PW) {
    bool any_pw = false;
#pragma unroll
    for (int J = 0; J < NB; ++J)
      any_pw = any_pw || pwf[J] != 0.f;
    if (threadIdx.x == 0)
      ba.pwflag[blockIdx.x] = any_pw ? 1 : 0;
    if (any_pw)
      return;  // the whole workgroup (the flags are uniform): the PW variant takes it
  }
  // S and dH in fragment layout `layout` (ST_::COL or ST_::ROW) to LDS: a
  // direct global -> LDS copy in 1 KB pieces (16 bytes a lane), the pieces
  // dealt to the waves in turn; waited for (vmcnt) and published by a
  // barrier before the first read
  const int wv = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  auto stage_states = [&](size_t layout) {
    if constexpr (L::STAGE) {
      constexpr int PIECES = static_cast<int>((2 * L::STB + 1023) / 1024);
#pragma unroll
      for (int i = 0; i < (PIECES + NB - 1) / NB; ++i) {
        const int pc = wv + NB * i;
        if (pc < PIECES) {
          const size_t o = static_cast<size_t>(pc) * 1024 + 16 * static_cast<size_t>(lane);
          const unsigned char *src = o < L::STB ? St + layout + o : Ht + layout + (o - L::STB);
          __builtin_amdgcn_global_load_lds(
              (const __attribute__((address_space(1))) void *)src,
              (__attribute__((address_space(3))) void *)(smb + L::STG + static_cast<size_t>(pc) * 1024), 16, 0, 0);
        }
      }
    }
  };
  auto staged_wait = [&]() {
    if constexpr (L::STAGE)
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  const unsigned char *sS = smb + L::STG, *sH = smb + L::STG + L::STB;  // staged S, dH tiles
  stage_states(ST_::COL);

  // Without PW every sub-block decays by at most e^-DIAG_LIM_LN, so every
  // cumulative log decay is finite and bounded (|g| <= C DIAG_LIM_LN / 16):
  // gv becomes the chunk's cumulative g_t and the factors are differences
  // of it.  With PW gv stays relative to the sub-block and every factor is
  // a sum (any decay, -inf included).
  if constexpr (!PW) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      if (I > 0)
        gv[kk] += rho_end(I - 1, kk);
  }
  // e^{rho_{I+1} - g_t}, the key's factor
  auto key_fac = [&](int kk) -> f32x4 {
    if constexpr (PW)
      return kfac[PW ? kk : 0];
    else
      return ex4(rho_end(I, kk) - gv[kk]);
  };
  // e^{g_t - rho_{J+1}} for J <= I (the row's side of pair (I, J))
  auto row_fac = [&](int J, int kk) -> f32x4 {
    if constexpr (PW)
      return ex4(J < I ? gv[kk] + tot_sum(J + 1, I, kk) : gv[kk] - tot_sum(I, I + 1, kk));
    else
      return ex4(gv[kk] - rho_end(J, kk));
  };
  // e^{g_t} and e^{g_C - g_t}
  auto start_fac = [&](int kk) -> f32x4 {
    if constexpr (PW)
      return ex4(gv[kk] + tot_sum(0, I, kk));
    else
      return ex4(gv[kk]);
  };
  auto end_fac = [&](int kk) -> f32x4 {
    if constexpr (PW)
      return kfac[PW ? kk : 0] * ex4(tot_sum(I + 1, NB, kk));
    else
      return ex4(rho_end(NB - 1, kk) - gv[kk]);
  };

  // ---- K~ rows to LDS, then A and P tiles (I, J <= I)
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
    stm_row(KT, PDL, 16 * I, 16 * kk, lane, kv[kk] * key_fac(kk));
  lds_barrier();
#pragma unroll
  for (int J = 0; J < NB; ++J) {
    if (J < I || (J == I && !PW)) {  // J unrolled: the decay sums become independent reads
      f32x4 aa = zero4, pp = zero4;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const f32x4 sc = row_fac(J, kk);
        const F kt = ldm_row(KT, PDL, 16 * J, 16 * kk, lane);
        mm_io(aa, F::from(ev[kk] * sc), kt);
        mm_io(pp, F::from(qv[kk] * sc), kt);
      }
      if (J == I) {
        aa = tri_col(aa, lane, true);
        pp = tri_col(pp, lane, false);
      }
      st_colf(sA, PC, 16 * I, 16 * J, lane, aa);
      stm_col(sP, PCL, 16 * I, 16 * J, lane, pp);
    }
  }
  if constexpr (PW) {
    // the diagonal pair, token by token (any decay, alpha = 0 included)
    f32x4 da, dp;
    wy_diag_pairwise<IO, D>(a, t0, len, h, I, lane, qs, ks, da, dp);
    st_rowf(sA, PC, 16 * I, 16 * I, lane, da);
    stm_row(sP, PCL, 16 * I, 16 * I, lane, dp);
  }
  staged_wait();  // S, dH (column layout) are in LDS after the barrier
  lds_barrier();

  // ---- diagonal blocks of T = (I + A)^{-1} (lane c < 16: column c), Y_I = U_I - ES_I S
  // w and v of every column are loaded first: they arrive during the solve
  raw4<IO> rw[NK], rv[NK];
#pragma unroll
  for (int n = 0; n < NK; ++n) {
    const int c0 = 16 * n + 4 * g;
    rw[n] = (GN && SWm) ? raw4<IO>::splat(w[srow]) : raw4<IO>::ld(w + row + c0);
    rv[n] = raw4<IO>::ld(v + row + c0);
  }
  if (lane < 16) {
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = (r == lane) ? 1.f : 0.f;
#pragma unroll
      for (int s2 = 0; s2 < r; ++s2)
        acc -= sA[(16 * I + r) * PC + 16 * I + s2] * x[s2];
      x[r] = acc;
      sT[(16 * I + r) * PC + 16 * I + lane] = acc;
    }
  }
  f32x4 zv[NK];  // Y, then Z
  {
    F esf[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      esf[kk] = F::from(ev[kk] * start_fac(kk));  // e e^{g_t}
    // S tiles from LDS (staged), or from global memory with the tiles of
    // column n + 1 loaded while column n is multiplied
    F cur[NK], nxt[NK];
    if constexpr (!L::STAGE) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        cur[kk] = F::ld(St + ST_::COL + ST_::off(kk, 0), lane);
    }
#pragma unroll
    for (int n = 0; n < NK; ++n) {
      if constexpr (L::STAGE) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          cur[kk] = F::ld(sS + ST_::off(kk, n), lane);
      } else if (n + 1 < NK) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          nxt[kk] = F::ld(St + ST_::COL + ST_::off(kk, n + 1), lane);
      }
      f32x4 acc = zero4;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        mm_io(acc, cur[kk], esf[kk]);
      if constexpr (!L::STAGE) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          cur[kk] = nxt[kk];
      }
      f32x4 u = ((GN && LPm) ? sig4(rw[n].f()) : rw[n].f()) * rv[n].f();
      zv[n] = (valid ? u : zero4) - acc;
      stm_row(YZ, PDL, 16 * I, 16 * n, lane, zv[n]);
    }
  }
  lds_barrier();
  // off-diagonal blocks of T, one block diagonal per round:
  // T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ
  for (int d = 1; d < NB; ++d) {
    if (I >= d) {
      const int J = I - d;
      f32x4 mk = zero4;
      for (int K = J; K < I; ++K)
        mm<float>(mk, ld_rowf(sA, PC, 16 * I, 16 * K, lane), ld_colf(sT, PC, 16 * K, 16 * J, lane));
      f32x4 tij = zero4;
      mm<float>(tij, ld_rowf(sT, PC, 16 * I, 16 * I, lane), mk);
      st_colf(sT, PC, 16 * I, 16 * J, lane, -tij);
    }
    lds_barrier();
  }

  // ---- Z_I = sum_{J <= I} T_IJ Y_J
#pragma unroll
  for (int n = 0; n < NK; ++n) {
    f32x4 acc = zero4;
    for (int J = 0; J <= I; ++J)
      mm_io(acc, ldm_col(YZ, PDL, 16 * J, 16 * n, lane), F::from(ld_rowf(sT, PC, 16 * I, 16 * J, lane)));
    zv[n] = acc;
  }
  f32x4 dov[NK];
#pragma unroll
  for (int n = 0; n < NK; ++n) {
    const f32x4 x = io<IO>::load4(dout + row + 16 * n + 4 * g);
    dov[n] = valid ? x : zero4;
  }
  lds_barrier();  // Y and A are no longer read
#pragma unroll
  for (int n = 0; n < NK; ++n) {
    stm_row(YZ, PDL, 16 * I, 16 * n, lane, zv[n]);
    stm_row(DOZ, PDL, 16 * I, 16 * n, lane, dov[n]);
  }
  lds_barrier();

  // ---- dZ_I = sum_{J >= I} P_JI^T dO_J + KB_I dH
  f32x4 dyv[NK];  // dZ, then dY
  {
    F kbf[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      kbf[kk] = F::from(kv[kk] * end_fac(kk));  // k e^{g_C - g_t}
    // dH tiles from LDS (staged), or from global memory with column n + 1 in
    // flight during column n
    F cur[NK], nxt[NK];
    if constexpr (!L::STAGE) {
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        cur[kk] = F::ld(Ht + ST_::COL + ST_::off(kk, 0), lane);
    }
#pragma unroll
    for (int n = 0; n < NK; ++n) {
      if constexpr (L::STAGE) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          cur[kk] = F::ld(sH + ST_::off(kk, n), lane);
      } else if (n + 1 < NK) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          nxt[kk] = F::ld(Ht + ST_::COL + ST_::off(kk, n + 1), lane);
      }
      f32x4 acc = zero4;
      for (int J = I; J < NB; ++J)
        mm_io(acc, ldm_col(DOZ, PDL, 16 * J, 16 * n, lane), ldm_col(sP, PCL, 16 * J, 16 * I, lane));
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        mm_io(acc, cur[kk], kbf[kk]);
      if constexpr (!L::STAGE) {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          cur[kk] = nxt[kk];
      }
      dyv[n] = acc;
    }
  }
  lds_barrier();  // dO of the other sub-blocks (and the staged column layouts) are no longer read
  // row layouts of S and dH, for dq, de, dk and d gamma_C: staged from the
  // stored copy, or (bfloat16 states carry the column layout only) re-laid
  // in place, each wave turning its share of the staged tiles from ColFrag
  // to RowFrag with one identity product per tile (exact)
  if constexpr (ST_::HAS_ROW) {
    stage_states(ST_::ROW);
  } else {
    static_assert(L::STAGE, "column-only states are read through the staged copy");
    constexpr int NTILE = 2 * NK * NK, PER = (NTILE + NB - 1) / NB, BATCH = PER < 8 ? PER : 8;
    const F eye = identity_colfrag<IO>(lane);
    unsigned char *stg = smb + L::STG;
#pragma unroll 1
    for (int r0 = 0; r0 < PER; r0 += BATCH) {
      F x[BATCH];
#pragma unroll
      for (int r = 0; r < BATCH; ++r) {
        const int p = wv + NB * (r0 + r);
        if (r0 + r < PER && p < NTILE)
          x[r] = F::ld(stg + static_cast<size_t>(p) * F::TILE_BYTES, lane);
      }
#pragma unroll
      for (int r = 0; r < BATCH; ++r) {
        const int p = wv + NB * (r0 + r);
        if (r0 + r < PER && p < NTILE)
          F::from(transpose_io(x[r], eye, lane)).st(stg + static_cast<size_t>(p) * F::TILE_BYTES, lane);
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NK; ++n)
    stm_row(DOZ, PDL, 16 * I, 16 * n, lane, dyv[n]);
  lds_barrier();
  // dY_I = sum_{J >= I} T_JI^T dZ_J;  dv = dY (.) w, dw = dY (.) v
  IO *dq = static_cast<IO *>(ba.dq), *dk = static_cast<IO *>(ba.dk), *db = static_cast<IO *>(ba.db);
  IO *dal = static_cast<IO *>(ba.dal), *dvo = static_cast<IO *>(ba.dv), *dwo = static_cast<IO *>(ba.dw);
  float dws = 0.f;  // dw summed over the channels (w per (token, head))
#pragma unroll
  for (int n = 0; n < NK; ++n) {
    const int c0 = 16 * n + 4 * g;
    rw[n] = (GN && SWm) ? raw4<IO>::splat(w[srow]) : raw4<IO>::ld(w + row + c0);
    rv[n] = raw4<IO>::ld(v + row + c0);
  }
#pragma unroll
  for (int n = 0; n < NK; ++n) {
    f32x4 acc = zero4;
    for (int J = I; J < NB; ++J)
      mm_io(acc, ldm_col(DOZ, PDL, 16 * J, 16 * n, lane), F::from(ld_colf(sT, PC, 16 * J, 16 * I, lane)));
    dyv[n] = acc;
    const int c0 = 16 * n + 4 * g;
    if constexpr (!GN) {
      if (valid) {
        io<IO>::store4(dvo + row + c0, acc * rw[n].f());
        io<IO>::store4(dwo + row + c0, acc * rv[n].f());
      }
    } else {
      const f32x4 wq = LPm ? sig4(rw[n].f()) : rw[n].f();
      f32x4 dwq = acc * rv[n].f();
      if (LPm)
        dwq *= wq * (f32x4{1.f, 1.f, 1.f, 1.f} - wq);  // through the sigmoid
      if (valid) {
        io<IO>::store4(dvo + row + c0, acc * wq);
        if (!SWm)
          io<IO>::store4(dwo + row + c0, dwq);
      }
      dws += (dwq[0] + dwq[1]) + (dwq[2] + dwq[3]);
    }
  }
  if constexpr (GN) {
    dws = row_sum(dws);
    if (SWm && valid && g == 0)
      dwo[srow] = io<IO>::from_f(dws);
  }

  // ---- dA_IJ = -dY_I Z_J^T, dP_IJ = dO_I Z_J^T (J <= I), as ColFrag (c) and RowFrag (r),
  // kept as operand fragments (every later use is a product operand)
  F dof[NK], dyf[NK], zf[NK];
#pragma unroll
  for (int n = 0; n < NK; ++n) {
    dof[n] = F::from(dov[n]);
    dyf[n] = F::from(dyv[n]);
    zf[n] = F::from(zv[n]);
  }
  F dAc[NB], dAr[NB], dPc[NB], dPr[NB];
#pragma unroll
  for (int J = 0; J < NB; ++J) {
    f32x4 ac = zero4, ar = zero4, pc = zero4, pr = zero4;
    if (J <= I) {
#pragma unroll
      for (int n = 0; n < NK; ++n) {
        const F zr = ldm_row(YZ, PDL, 16 * J, 16 * n, lane);
        mm_io(ac, dyf[n], zr);
        mm_io(ar, zr, dyf[n]);
        mm_io(pc, dof[n], zr);
        mm_io(pr, zr, dof[n]);
      }
      ac = -ac;
      ar = -ar;
      if (J == I) {
        ac = tri_col(ac, lane, true);
        pc = tri_col(pc, lane, false);
        ar = tri_row(ar, lane, true);
        pr = tri_row(pr, lane, false);
      }
    }
    dAc[J] = F::from(ac);
    dAr[J] = F::from(ar);
    dPc[J] = F::from(pc);
    dPr[J] = F::from(pr);
  }
  if constexpr (PW) {
    // this sub-block's diagonal dA, dP (row t = m, columns 4g .. 4g+3), for
    // the pairwise gradients below (read by this wave only)
    float *dA_I = diag + I * 512, *dP_I = dA_I + 256;
    *reinterpret_cast<f32x4 *>(dA_I + m * 16 + 4 * g) = dAr[I].to_f32();
    *reinterpret_cast<f32x4 *>(dP_I + m * 16 + 4 * g) = dPr[I].to_f32();
  }

  // ---- contributions to dq (cq), de (ce), dk (ck) and d g_C (kb term)
  f32x4 cq[NK], ce[NK], ck[NK];
  // S and dH tiles in row layout: from LDS (staged; waited for here), or from
  // global memory with row tile kk + 1 loaded while row tile kk is multiplied
  F scur[NK], hcur[NK], snxt[NK], hnxt[NK];
  if constexpr (L::STAGE) {
    staged_wait();
    lds_barrier();
  } else {
#pragma unroll
    for (int n = 0; n < NK; ++n) {
      scur[n] = F::ld(St + ST_::ROW + ST_::off(0, n), lane);
      hcur[n] = F::ld(Ht + ST_::ROW + ST_::off(0, n), lane);
    }
  }
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    if constexpr (L::STAGE) {
#pragma unroll
      for (int n = 0; n < NK; ++n) {
        scur[n] = F::ld(sS + ST_::off(kk, n), lane);
        hcur[n] = F::ld(sH + ST_::off(kk, n), lane);
      }
    } else if (kk + 1 < NK) {
#pragma unroll
      for (int n = 0; n < NK; ++n) {
        snxt[n] = F::ld(St + ST_::ROW + ST_::off(kk + 1, n), lane);
        hnxt[n] = F::ld(Ht + ST_::ROW + ST_::off(kk + 1, n), lane);
      }
    }
    f32x4 a1 = zero4, a2 = zero4, a3 = zero4;
#pragma unroll
    for (int n = 0; n < NK; ++n) {
      mm_io(a1, scur[n], dof[n]);
      mm_io(a2, scur[n], dyf[n]);
      mm_io(a3, hcur[n], zf[n]);
    }
    if constexpr (!L::STAGE) {
#pragma unroll
      for (int n = 0; n < NK; ++n) {
        scur[n] = snxt[n];
        hcur[n] = hnxt[n];
      }
    }
    const f32x4 eg = start_fac(kk);  // e^{g_t}
    cq[kk] = a1 * eg;
    ce[kk] = -(a2 * eg);
    ck[kk] = a3 * end_fac(kk);  // dKB e^{g_C - g}
#pragma unroll
    for (int J = 0; J < NB; ++J) {
      if (J < I || (J == I && !PW)) {
        const F ktc = ldm_col(KT, PDL, 16 * J, 16 * kk, lane);
        f32x4 aq = zero4, ae = zero4;
        mm_io(aq, ktc, dPr[J]);
        mm_io(ae, ktc, dAr[J]);
        const f32x4 sc = row_fac(J, kk);
        cq[kk] += aq * sc;
        ce[kk] += ae * sc;
      }
    }
    if constexpr (PW) {
      // the diagonal pair: dq_t += sum_s dP_ts k_s F_ts, de_t += sum_s dA_ts k_s F_ts
      // over s = t - j of this sub-block, F_ts = alpha_t .. alpha_{s+1}
      f32x4 q4, k4, e4, a4;
      wy_row4<IO, D>(a, srow, valid, 16 * kk + 4 * g, qs, ks, q4, k4, e4, a4);
      const float *dA_I = diag + I * 512, *dP_I = dA_I + 256;
      f32x4 Fp = {1.f, 1.f, 1.f, 1.f}, xq = zero4, xe = zero4;
#pragma unroll 1
      for (int j = 0; j < 16; ++j) {
        const int src = m >= j ? lane - j : lane, srca = m >= j ? lane - j + 1 : lane;
        f32x4 kf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (j > 0)
            Fp[i] *= __shfl(a4[i], srca, 64);
          kf[i] = __shfl(k4[i], src, 64) * Fp[i];
        }
        if (m >= j) {
          xq += kf * dP_I[m * 16 + (m - j)];
          if (j > 0)
            xe += kf * dA_I[m * 16 + (m - j)];
        }
      }
      cq[kk] += xq;
      ce[kk] += xe;
    }
  }

  // ---- dK~_J contributions of this sub-block's rows, one LDS slot per
  // (I, J <= I); the owner of J sums its slots in ascending I (a fixed order)
  f32x4 qrc[NK], erc[NK];  // ColFrag of q e^{g - rho_I} and e e^{g - rho_I}
  {
    raw4<IO> rq[NK], rk[NK], rb[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int c0 = 16 * kk + 4 * g;
      rq[kk] = raw4<IO>::ld(q + row + c0);
      rk[kk] = raw4<IO>::ld(k + row + c0);
      if constexpr (!GN)
        rb[kk] = raw4<IO>::ld(b + row + c0);
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      // PW: e^{g_t - rho_I} (column factors from rho_I); else e^{g_t - rho_{I+1}}
      const f32x4 sc = valid ? (PW ? ex4(gv[kk]) : ex4(gv[kk] - rho_end(I, kk))) : zero4;
      const f32x4 bq = GN ? ld_b(16 * kk + 4 * g) : rb[kk].f();
      qrc[kk] = transpose_f32(rq[kk].f() * (qs * sc), lane);
      erc[kk] = transpose_f32(bq * rk[kk].f() * (ks * sc), lane);
    }
  }
  lds_barrier();  // K~, T, P, Y/Z and dZ are no longer read: the dK~ sums take the bottom of the LDS
  // dK~_J = sum over the sub-blocks I >= J of their rows' terms, added in
  // ascending I: in round r wave I adds its term for J = I - r (round 0
  // writes it), so every sum is formed in the same order on every run.
  auto dk_sum = [&](int J2, int kk) { return reinterpret_cast<f32x4 *>(smb + L::DKS) + (J2 * NK + kk) * 64; };
  {
    // column scale of ColFrag element (lane column c): e^{rho_I - rho_{J+1}}
    // (the sub-blocks between J and I, summed up while J descends), and
    // e^{-(sub-block I's log decay)} for the diagonal pair
    float rs[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      rs[kk] = 0.f;
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      const int J = I - r;
      if (J >= 0) {
        F dpj = dPc[0], daj = dAc[0];  // dP_IJ, dA_IJ (selected, not indexed: they stay in registers)
#pragma unroll
        for (int J2 = 1; J2 < NB; ++J2)
          if (J2 == J) {
            dpj = dPc[J2];
            daj = dAc[J2];
          }
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          f32x4 acc = zero4;
          if constexpr (PW) {
            // e^{rho_I - rho_{J+1}} for J < I; the diagonal pair is added below
            if (J < I - 1)
              rs[kk] += btot[(J + 1) * D + 16 * kk + m];
            if (J < I) {
              const float f = __expf(rs[kk]);
              mm_io(acc, F::from(qrc[kk] * f), dpj);
              mm_io(acc, F::from(erc[kk] * f), daj);
            }
          } else {
            // e^{rho_{I+1} - rho_{J+1}}
            if (J < I)
              rs[kk] += btot[(J + 1) * D + 16 * kk + m];
            const float f = __expf(rs[kk]);
            mm_io(acc, F::from(qrc[kk] * f), dpj);
            mm_io(acc, F::from(erc[kk] * f), daj);
          }
          f32x4 *ps = dk_sum(J, kk) + lane;
          *ps = (r == 0) ? acc : *ps + acc;
        }
      }
      lds_barrier();
    }
  }

  // ---- map to the inputs
  // d gamma_C = rowsum(dH (.) S): wave I takes row tiles kk = I, I + NB, ..
  if constexpr (L::STAGE) {
    // staged row layout: lane (m, g) of RowFrag tile (kk, n) holds row
    // 16kk + m, columns 16n + 4g .. +3
    for (int kk = I; kk < NK; kk += NB) {
      float x = 0.f;
#pragma unroll
      for (int n = 0; n < NK; ++n) {
        const f32x4 p = F::ld(sS + ST_::off(kk, n), lane).to_f32() * F::ld(sH + ST_::off(kk, n), lane).to_f32();
        x += (p[0] + p[1]) + (p[2] + p[3]);
      }
      x += __shfl_xor(x, 16, 64);
      x += __shfl_xor(x, 32, 64);
      if (g == 0)
        dgam[16 * kk + m] = x;
    }
  } else {
    // lane (c, g) of ColFrag tile (kk, n) holds rows 16kk + 4g .. +3 of column 16n + c
    for (int kk = I; kk < NK; kk += NB) {
      f32x4 acc = zero4;
#pragma unroll
      for (int n = 0; n < NK; ++n)
        acc += F::ld(St + ST_::COL + ST_::off(kk, n), lane).to_f32() *
               F::ld(Ht + ST_::COL + ST_::off(kk, n), lane).to_f32();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = acc[i];
        x += __shfl_xor(x, 1, 16);
        x += __shfl_xor(x, 2, 16);
        x += __shfl_xor(x, 4, 16);
        x += __shfl_xor(x, 8, 16);
        acc[i] = x;
      }
      if (m == 0)
        *reinterpret_cast<f32x4 *>(dgam + 16 * kk + 4 * g) = acc;
    }
  }
  f32x4 dg[NK];
  raw4<IO> ral[NK];  // alpha of the rows, for d alpha at the end
  if constexpr (!GN) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      ral[kk] = raw4<IO>::ld(al + row + 16 * kk + 4 * g);
  }
  // q, k, b of row tile kk + 1 are loaded while tile kk is mapped
  raw4<IO> nq = raw4<IO>::ld(q + row + 4 * g), nk = raw4<IO>::ld(k + row + 4 * g), nb;
  if constexpr (!GN)
    nb = raw4<IO>::ld(b + row + 4 * g);
  float dotq = 0.f, dotk = 0.f, dbs = 0.f;  // GN: row sums for layer prep and per-(token, head) b
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    f32x4 ckt = dk_sum(I, kk)[lane] * key_fac(kk);
    if constexpr (PW) {
      // the diagonal pair: dk_s += sum_t (dP_ts q_t + dA_ts e_t) F_ts over
      // t = s + j of this sub-block, F_ts = alpha_{s+1} .. alpha_t
      f32x4 q4, k4, e4, a4;
      wy_row4<IO, D>(a, srow, valid, 16 * kk + 4 * g, qs, ks, q4, k4, e4, a4);
      const float *dA_I = diag + I * 512, *dP_I = dA_I + 256;
      f32x4 Fk = {1.f, 1.f, 1.f, 1.f};
#pragma unroll 1
      for (int j = 0; j < 16; ++j) {
        const int src = m + j <= 15 ? lane + j : lane;
        f32x4 qt, et;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (j > 0)
            Fk[i] *= __shfl(a4[i], src, 64);
          qt[i] = __shfl(q4[i], src, 64);
          et[i] = __shfl(e4[i], src, 64);
        }
        if (m + j <= 15) {
          const int tt = m + j;
          ckt += (qt * dP_I[tt * 16 + m] + (j > 0 ? et * dA_I[tt * 16 + m] : zero4)) * Fk;
        }
      }
    }
    const int c0 = 16 * kk + 4 * g;
    f32x4 qq = nq.f() * qs, kq = nk.f() * ks, bq = GN ? ld_b(c0) : nb.f();
    if (!valid)
      qq = kq = bq = zero4;
    if (kk + 1 < NK) {
      nq = raw4<IO>::ld(q + row + c0 + 16);
      nk = raw4<IO>::ld(k + row + c0 + 16);
      if constexpr (!GN)
        nb = raw4<IO>::ld(b + row + c0 + 16);
    }
    const f32x4 kbt = kq * ck[kk];  // k (.) dKB-contribution, part of d g_C
    dg[kk] = qq * cq[kk] + bq * kq * ce[kk] - kq * (ck[kk] + ckt);
    if constexpr (!GN) {
      if (valid) {
        io<IO>::store4(dq + row + c0, cq[kk]);
        io<IO>::store4(dk + row + c0, ck[kk] + ckt + bq * ce[kk]);
        io<IO>::store4(db + row + c0, kq * ce[kk]);
      }
    } else {
      // gradients with respect to the recurrence's k and b, kept for the
      // second pass (ck, ce are not read again otherwise)
      ck[kk] = ck[kk] + ckt + bq * ce[kk];
      ce[kk] = kq * ce[kk];
      if (LPm)
        ce[kk] *= bq * (f32x4{1.f, 1.f, 1.f, 1.f} - bq);  // through the sigmoid
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dotq += qq[i] * cq[kk][i];
        dotk += kq[i] * ck[kk][i];
        dbs += ce[kk][i];
      }
    }
    // sub-block sums over the 16 rows: kb terms and dg
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float kbsc = row16_inclusive_scan(kbt[i]);
      const float gs = row16_inclusive_scan(dg[kk][i]);
      if (m == 15) {
        kbs[I * D + c0 + i] = kbsc;
        gtot[I * D + c0 + i] = gs;
      }
      dg[kk][i] = gs;  // in-block inclusive prefix of dg
    }
  }
  if constexpr (GN) {
    // second pass: through the L2 normalisation (layer prep),
    // dx = (dq - q (q . dq)) / |x|, and the stores
    dotq = row_sum(dotq);
    dotk = row_sum(dotk);
    dbs = row_sum(dbs);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int c0 = 16 * kk + 4 * g;
      f32x4 dqv = cq[kk], dkv = ck[kk];
      if (LPm) {
        const f32x4 qh = raw4<IO>::ld(q + row + c0).f() * qs, kh = raw4<IO>::ld(k + row + c0).f() * ks;
        dqv = (dqv - qh * dotq) * qs;
        dkv = (dkv - kh * dotk) * ks;
      }
      if (valid) {
        io<IO>::store4(dq + row + c0, dqv);
        io<IO>::store4(dk + row + c0, dkv);
        if (!SBm)
          io<IO>::store4(db + row + c0, ce[kk]);
      }
    }
    if (SBm && valid && g == 0)
      db[srow] = io<IO>::from_f(dbs);
  }
  lds_barrier();
  // d ln(alpha_t) = sum_{s >= t} dg_s + d g_C, d g_C = gamma dgamma + sum of the kb terms
  float das = 0.f;  // GN: d alpha summed over the channels
#pragma unroll
  for (int kk = 0; kk < NK; ++kk) {
    const int c0 = 16 * kk + 4 * g;
    const f32x4 gc = rho_end(NB - 1, kk);
    const f32x4 own = *reinterpret_cast<const f32x4 *>(gtot + I * D + c0);
    f32x4 tail = zero4, kbsum = zero4;
    for (int J = 0; J < NB; ++J) {
      kbsum += *reinterpret_cast<const f32x4 *>(kbs + J * D + c0);
      if (J > I)
        tail += *reinterpret_cast<const f32x4 *>(gtot + J * D + c0);
    }
    const f32x4 dgc = ex4(gc) * *reinterpret_cast<const f32x4 *>(dgam + c0) + kbsum;
    // suffix within the sub-block: total - inclusive prefix + own element
    f32x4 mine;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float prev = __shfl_up(dg[kk][i], 1, 16);
      mine[i] = dg[kk][i] - (m == 0 ? 0.f : prev);
    }
    const f32x4 dl = own - dg[kk] + mine + tail + dgc;
    if constexpr (!GN) {
      if (valid)
        io<IO>::store4(dal + row + c0, dl / ral[kk].f());
    } else {
      // layer prep: the input is ln(alpha) (float32), whose gradient is dl
      const f32x4 da = LPm ? dl : dl / ld_alpha(c0);
      if (valid && !SAm) {
        if (LPm)
          *reinterpret_cast<f32x4 *>(static_cast<float *>(ba.dal) + row + c0) = da;
        else
          io<IO>::store4(dal + row + c0, da);
      }
      das += (da[0] + da[1]) + (da[2] + da[3]);
    }
  }
  if constexpr (GN) {
    das = row_sum(das);
    if (SAm && valid && g == 0) {
      if (LPm)
        static_cast<float *>(ba.dal)[srow] = das;
      else
        dal[srow] = io<IO>::from_f(das);
    }
  }
}

template <typename IO, int D, int C> hipError_t launch_bwd_dstate(const bwd_args &a, hipStream_t st) {
  const long units_pad = (static_cast<long>(a.f.num_seqs) * a.f.H + 7) / 8 * 8;
  hipLaunchKernelGGL((gdn2_bwd_dstate_kernel<IO, D, C>), dim3(static_cast<unsigned>(units_pad * dstate_cfg<D>::NSPL)),
                     dim3(64 * dstate_cfg<D>::NW), 0, st, a);
  return hipGetLastError();
}

// Two launches: every chunk-head whose decays allow the matrix-core
// diagonal, then the PW variant on the rest (flags from the first).
template <typename IO, int D, int C, bool PW> hipError_t launch_bwd_grad_pass(const bwd_args &a, hipStream_t st) {
  const long n = static_cast<long>(a.f.num_slots) * a.f.H;
  const dim3 grid(static_cast<unsigned>(n)), block(64 * (C / 16));
  const uint32_t kda = GATE_SCALAR_B | GATE_SCALAR_W, gdn = kda | GATE_SCALAR_ALPHA;
  if constexpr (PW) {
    // the rare path: one variant that reads every input layout from the flags
    (void)kda;
    (void)gdn;
    hipLaunchKernelGGL((gdn2_bwd_grad_kernel<IO, D, C, IO, BG_FLAGS, true>), grid, block, 0, st, a);
  } else {
    if (a.f.gates == 0)
      hipLaunchKernelGGL((gdn2_bwd_grad_kernel<IO, D, C, IO, BG_PLAIN, false>), grid, block, 0, st, a);
    else if (a.f.gates == kda)
      hipLaunchKernelGGL((gdn2_bwd_grad_kernel<IO, D, C, IO, BG_KDA, false>), grid, block, 0, st, a);
    else if (a.f.gates == gdn)
      hipLaunchKernelGGL((gdn2_bwd_grad_kernel<IO, D, C, IO, BG_GDN, false>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((gdn2_bwd_grad_kernel<IO, D, C, IO, BG_FLAGS, false>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <typename IO, int D, int C> hipError_t launch_bwd_grad(const bwd_args &a, hipStream_t st) {
  const hipError_t e = launch_bwd_grad_pass<IO, D, C, false>(a, st);
  if (e != hipSuccess)
    return e;
  return launch_bwd_grad_pass<IO, D, C, true>(a, st);
}

#define GDN2_INST_BWD(IO, D, C)                                                    \
  template hipError_t launch_bwd_dstate<IO, D, C>(const bwd_args &, hipStream_t); \
  template hipError_t launch_bwd_grad<IO, D, C>(const bwd_args &, hipStream_t);

GDN2_INST_BWD(float, 16, 16)
GDN2_INST_BWD(float, 32, 16)
GDN2_INST_BWD(float, 64, 16)
GDN2_INST_BWD(float, 128, 16)
GDN2_INST_BWD(float, 16, 64)
GDN2_INST_BWD(float, 32, 64)
GDN2_INST_BWD(float, 64, 64)
GDN2_INST_BWD(float, 128, 64)
GDN2_INST_BWD(bf16_t, 16, 16)
GDN2_INST_BWD(bf16_t, 32, 16)
GDN2_INST_BWD(bf16_t, 64, 16)
GDN2_INST_BWD(bf16_t, 128, 16)
GDN2_INST_BWD(bf16_t, 16, 64)
GDN2_INST_BWD(bf16_t, 32, 64)
GDN2_INST_BWD(bf16_t, 64, 64)
GDN2_INST_BWD(bf16_t, 128, 64)

}  // namespace gdn2
