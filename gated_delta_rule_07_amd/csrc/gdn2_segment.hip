// gdn2_segment.hip -- the state map of a sequence segment, and its composition
// (gfx950).
//
// Over one segment (any run of chunks), the state recurrence of the chunked
// forward is affine in the entering state:
//   S_out = Phi S_in + Psi,
// with Phi (dk x dk) the product over the segment's chunks, last first, of
// Diag(gamma_C) - Kbar^T W, and Psi (dk x dv) the state after the segment
// when it starts from zero.  Phi is the same recurrence run on an identity
// entering state with the values (Ut) left out.  A long sequence cut into
// segments then needs only the segments' maps to find every segment's true
// entering state (an exclusive scan of (Phi, Psi) pairs), after which each
// segment runs on its own.  This is the context-parallel split of the
// sequence axis: each GPU would own segments, and the scan of the maps is the
// one exchange.  Here both steps run on one GPU:
//   gdn2_segmap_kernel      (Psi, Phi) of every (segment, head), each segment
//                           being one sequence of a (packed) batch;
//   gdn2_seg_combine_kernel the exclusive scan over the segments of one
//                           sequence: S_in(0) = S0, S_in(g+1) = Phi_g S_in(g) + Psi_g.
#include "gdn2_kernels.hpp"
#include "gdn2_wy.hpp"

namespace gdn2 {

// Workgroups per (segment, head) and map: NSPL, each with NW = NK / NSPL
// compute waves, one per 16-column tile of the map; part 0 computes Psi,
// part 1 Phi.  Per chunk every compute wave takes
//   Z = [Ut] - W S,   S <- Diag(gamma_C) S + Kbar^T Z
// on its columns (Ut only for Psi) from the chunk's -W and Kbar^T tiles,
// its Ut tiles and gamma_C, staged in LDS: the -W and Kbar^T regions of the
// prep's block are copied byte for byte (16 or 8 bytes a lane), so
// they keep the block's tile order, with 16-wide k tiles paired; bfloat16
// products then take two k tiles per 16x16x32 instruction.
// bfloat16: NL loader waves stage the chunks into two LDS buffers, chunk k
// by loader (k - 1) mod NL, which issues its loads NL chunks before they
// are due, so the compute waves never wait on global memory (one barrier
// per chunk).  float32: the compute waves stage the tiles themselves, one
// chunk ahead (the loaders' registers would not hold float32 chunks).  More
// workgroups with fewer compute waves spread a few long segments over more
// compute units (the per-rank shape of a context-parallel split has only H
// units); every workgroup of one (segment, head) sits on the same XCD,
// whose L2 serves their common reads.
// Grid: units_pad * 2 * NSPL workgroups, units_pad = N*H rounded up to 8.
template <typename IO, int D, int C> struct segmap_cfg {
  static constexpr int NK = D / 16, NB = C / 16;
  static constexpr bool PIPE = sizeof(IO) == 2;
  static constexpr int NSPL = (PIPE && NK >= 4) ? NK / 2 : 1;
  static constexpr int NW = NK / NSPL;  // compute waves
  static constexpr int NL = PIPE ? 2 : 0;
  static constexpr int NBUF = PIPE ? 2 : 1;
  static constexpr size_t TB = frag<IO>::TILE_BYTES;
  static constexpr size_t RB = static_cast<size_t>(NB) * NK * TB;  // bytes of the -W region, and of Kbar^T's
  static constexpr int PW = RB % 1024 == 0 ? 16 : 8;                // bytes a lane copies per piece
  static constexpr size_t PB = 64 * PW;                              // bytes of one piece
  static constexpr int NRP = static_cast<int>(2 * RB / PB);          // pieces of the two regions
  static constexpr size_t UTO = 2 * RB, GMO = 2 * RB + NW * NB * TB;  // Ut tiles, gamma_C
  static constexpr size_t BUF = GMO + D * sizeof(float);
};

template <typename IO, int D, int C>
__global__ void __launch_bounds__((64 * (segmap_cfg<IO, D, C>::NW + segmap_cfg<IO, D, C>::NL)))
    gdn2_segmap_kernel(chunk_args a, float *Phi, float *Psi) {
  typedef segmap_cfg<IO, D, C> K;
  constexpr int NB = C / 16, NK = D / 16, NW = K::NW, NSPL = K::NSPL, NL = K::NL, NRP = K::NRP;
  typedef frag<IO> F;
  typedef frag2<IO> F2;
  typedef blk_layout<IO, D, C> L;
  typedef __attribute__((ext_vector_type(K::PW / 4))) unsigned int PV;  // one lane's share of a piece
  constexpr size_t TB = K::TB, RB = K::RB, PB = K::PB;
  constexpr int PW = K::PW;
  static_assert(RB % PB == 0, "each region is whole pieces");
  __shared__ __attribute__((aligned(16))) unsigned char sbuf[K::NBUF][K::BUF];

  const int x = blockIdx.x;
  const int xcd = x & 7, s8 = x >> 3;
  const int unit = (s8 / (2 * NSPL)) * 8 + xcd;
  const int part = (s8 % (2 * NSPL)) / NSPL, grp = s8 % NSPL;
  if (unit >= a.num_seqs * a.H)
    return;  // whole workgroup
  const int n = unit / a.H, h = unit - n * a.H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  int c_begin, nchunks;
  if (a.cu) {
    c_begin = a.offsets[n];
    nchunks = a.offsets[n + 1] - c_begin;
  } else {
    const int nc = (a.T + C - 1) / C;
    c_begin = n * nc;
    nchunks = nc;
  }
  const int last = nchunks - 1;  // loads past the end re-read the last chunk: no branch
  auto blk_of = [&](int c) {
    return reinterpret_cast<const unsigned char *>(a.blocks) +
           (static_cast<size_t>(c_begin + c) * a.H + h) * a.blk_bytes;
  };
  // this lane's PW bytes of region piece q in the block (LDS: q PB + PW lane)
  auto piece_src = [&](int q) -> size_t {
    return (q < NRP / 2 ? L::WN + static_cast<size_t>(q) * PB : L::KB + static_cast<size_t>(q - NRP / 2) * PB) +
           static_cast<size_t>(lane) * PW;
  };
  // this lane's fragment of Ut tile tt of compute wave w, in the block
  auto ut_src = [&](int w, int tt) -> size_t { return L::UT + tile_off<IO, NK>(tt, grp * NW + w, lane); };

  if constexpr (NL > 0) {
    if (wave >= NW) {
      // ---- loader wave: chunks 1 + l, 1 + l + NL, ...
      if (nchunks == 0)
        return;  // no barrier is taken
      const int l = wave - NW;
      constexpr int GPL = (D + 63) / 64;  // gamma entries per lane
      PV r[NRP];
      F u[NW * NB];
      float gv[GPL];
      auto gload = [&](int c) {
        const unsigned char *blk = blk_of(c);
#pragma unroll
        for (int q = 0; q < NRP; ++q)
          r[q] = *reinterpret_cast<const PV *>(blk + piece_src(q));
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int tt = 0; tt < NB; ++tt)
            u[w * NB + tt] = F::ld_at(blk + ut_src(w, tt));
#pragma unroll
        for (int q = 0; q < GPL; ++q)
          gv[q] = reinterpret_cast<const float *>(blk + L::GAM)[lane + 64 * q < D ? lane + 64 * q : D - 1];
      };
      auto lstore = [&](int b) {
#pragma unroll
        for (int q = 0; q < NRP; ++q)
          *reinterpret_cast<PV *>(&sbuf[b][q * PB + lane * PW]) = r[q];
#pragma unroll
        for (int i = 0; i < NW * NB; ++i)
          u[i].st(&sbuf[b][K::UTO + i * TB], lane);
#pragma unroll
        for (int q = 0; q < GPL; ++q)
          if (lane + 64 * q < D)
            reinterpret_cast<float *>(&sbuf[b][K::GMO])[lane + 64 * q] = gv[q];
      };
      if (l == 0) {
        gload(0);
        lstore(0);
      }
      gload(l + 1 < last ? l + 1 : last);
      lds_barrier();
      for (int i = 0; i < nchunks; ++i) {
        if (i % NL == l && i + 1 < nchunks) {
          lstore((i + 1) % 2);
          gload(i + 1 + NL < last ? i + 1 + NL : last);
        }
        lds_barrier();  // chunk i + 1 is staged, chunk i's buffer is free
      }
      return;
    }
  }

  // ---- compute wave: column tile j of the map
  const int j = grp * NW + wave;
  f32x4 s[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s[kk][i] = (part == 1 && kk == j && 4 * g + i == m) ? 1.f : 0.f;

  // the products of one chunk from its staged buffer
  constexpr bool PAIR_K = sizeof(IO) == 2 && NK % 2 == 0, PAIR_T = sizeof(IO) == 2 && NB % 2 == 0;
  auto step = [&](const unsigned char *sb) {
    F sf[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      sf[kk] = F::from(s[kk]);
    F zf[NB];
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
      f32x4 z = (part == 0) ? F::ld(sb + K::UTO + (wave * NB + tt) * TB, lane).to_f32() : f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (PAIR_K) {
#pragma unroll
        for (int kp = 0; kp < NK / 2; ++kp)
          mma32(z, F2::ld(sb + tile_off<IO, NK>(tt, 2 * kp, 0), lane), F2::make(sf[2 * kp], sf[2 * kp + 1]));
      } else {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
          mm_io(z, F::ld_at(sb + tile_off<IO, NK>(tt, kk, lane)), sf[kk]);
      }
      zf[tt] = F::from(z);
    }
    const float *gam = reinterpret_cast<const float *>(sb + K::GMO);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      s[kk] *= *reinterpret_cast<const f32x4 *>(gam + 16 * kk + 4 * g);
      if constexpr (PAIR_T) {
#pragma unroll
        for (int tp = 0; tp < NB / 2; ++tp)
          mma32(s[kk], F2::ld(sb + RB + tile_off<IO, NB>(kk, 2 * tp, 0), lane), F2::make(zf[2 * tp], zf[2 * tp + 1]));
      } else {
#pragma unroll
        for (int tt = 0; tt < NB; ++tt)
          mm_io(s[kk], F::ld_at(sb + RB + tile_off<IO, NB>(kk, tt, lane)), zf[tt]);
      }
    }
  };

  if (nchunks > 0) {
    if constexpr (NL > 0) {
      lds_barrier();
      for (int i = 0; i < nchunks; ++i) {
        step(sbuf[i % 2]);
        lds_barrier();
      }
    } else {
      // stage this wave's share of the pieces itself, one chunk ahead
      static_assert(64 * NW >= D, "one thread per gamma entry");
      constexpr int PPW = (NRP + NW - 1) / NW;
      PV r[PPW];
      F u[NB];
      float gv = 0.f;
      auto issue = [&](int c) {
        const unsigned char *blk = blk_of(c);
#pragma unroll
        for (int i = 0; i < PPW; ++i) {
          const int q = wave + i * NW;
          r[i] = *reinterpret_cast<const PV *>(blk + piece_src(q < NRP ? q : NRP - 1));
        }
#pragma unroll
        for (int tt = 0; tt < NB; ++tt)
          u[tt] = F::ld_at(blk + ut_src(wave, tt));
        gv = reinterpret_cast<const float *>(blk + L::GAM)[threadIdx.x < D ? threadIdx.x : D - 1];
      };
      auto commit = [&]() {
#pragma unroll
        for (int i = 0; i < PPW; ++i)
          if (wave + i * NW < NRP)
            *reinterpret_cast<PV *>(&sbuf[0][(wave + i * NW) * PB + lane * PW]) = r[i];
#pragma unroll
        for (int tt = 0; tt < NB; ++tt)
          u[tt].st(&sbuf[0][K::UTO + (wave * NB + tt) * TB], lane);
        if (threadIdx.x < D)
          reinterpret_cast<float *>(&sbuf[0][K::GMO])[threadIdx.x] = gv;
      };
      issue(0);
      commit();
      lds_barrier();
      for (int c = 0; c < nchunks; ++c) {
        issue(c + 1 < last ? c + 1 : last);
        step(sbuf[0]);
        lds_barrier();  // this chunk's tiles are no longer read
        if (c + 1 < nchunks)
          commit();
        lds_barrier();
      }
    }
  }
  float *out = (part == 0 ? Psi : Phi) + static_cast<size_t>(unit) * D * D;
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[(16 * kk + 4 * g + i) * D + 16 * j + m] = s[kk][i];
}

// One workgroup per (sequence, head, 16-column tile j of the state), one
// wave per 16-row tile kk.  B sequences of G segments each, maps
// [B][G][H][D][D] (segment g of sequence b at b G + g), S0 [B][H][D][D]:
// writes the state entering every segment to S_in [B][G][H][D][D] and, if
// S_final is given, the state after the last one, [B][H][D][D].  Per segment the column
// of state tiles (., j) sits in LDS and wave kk forms its tile of
// Psi_g + Phi_g S from row tile kk of Phi_g, loaded one segment ahead.
// float32 throughout (products as in mm<float>).
// REV: the adjoint scan of the backward, segments from the last: the input
// in S0's place is the gradient of the state after the last segment; then
// per segment g (descending) S_in[g] is the gradient of the state after g and
// the next one is Phi_g^T S_in[g] + Psi_g, with Psi_g the gradient of the
// state before g from g's own outputs; S_final receives the gradient of the
// state before the first segment.
template <int D, bool REV = false>
__global__ void __launch_bounds__(64 * (D / 16)) gdn2_seg_combine_kernel(const float *__restrict__ Phi,
                                                                         const float *__restrict__ Psi,
                                                                         const float *__restrict__ S0, int G, int H,
                                                                         int B, float *__restrict__ S_in,
                                                                         float *__restrict__ S_final) {
  constexpr int NK = D / 16;
  __shared__ f32x4 col[NK][64];  // ColFrag of the state tiles (k2, j)
  const int bh = static_cast<int>(blockIdx.x) / NK, j = static_cast<int>(blockIdx.x) % NK;
  if (bh >= B * H)
    return;
  const int b = bh / H, h = bh - b * H;
  // maps and entering states of sequence b: segment g is row b G + g; its
  // head h is then at ((b G + g) H + h), i.e. at (g H' + h) from Phi_b
  // with H' = H
  Phi += static_cast<size_t>(b) * G * H * D * D;
  Psi += static_cast<size_t>(b) * G * H * D * D;
  S_in += static_cast<size_t>(b) * G * H * D * D;
  const int kk = static_cast<int>(threadIdx.x) >> 6, lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  // element i of this lane's ColFrag of tile (kk, j) within one D x D matrix
  auto at = [&](int i) { return static_cast<size_t>(16 * kk + 4 * g + i) * D + 16 * j + m; };
  f32x4 s;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    s[i] = S0 ? S0[static_cast<size_t>(bh) * D * D + at(i)] : 0.f;
  f32x4 ph[NK], ps;  // RowFrag of Phi (REV: Phi^T) tiles (kk, k2); ColFrag of Psi tile (kk, j)
  auto load = [&](int seg) {
    const size_t base = (static_cast<size_t>(seg) * H + h) * D * D;
#pragma unroll
    for (int k2 = 0; k2 < NK; ++k2) {
      if constexpr (REV) {
        // Phi^T[16 kk + m][16 k2 + 4 g + i] = Phi[16 k2 + 4 g + i][16 kk + m]
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ph[k2][i] = Phi[base + static_cast<size_t>(16 * k2 + 4 * g + i) * D + 16 * kk + m];
      } else {
        ph[k2] = *reinterpret_cast<const f32x4 *>(Phi + base + static_cast<size_t>(16 * kk + m) * D + 16 * k2 + 4 * g);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ps[i] = Psi[base + at(i)];
  };
  if (G > 0)
    load(REV ? G - 1 : 0);
  for (int step = 0; step < G; ++step) {
    const int seg = REV ? G - 1 - step : step;
    const size_t base = (static_cast<size_t>(seg) * H + h) * D * D;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S_in[base + at(i)] = s[i];
    col[kk][lane] = s;
    lds_barrier();
    f32x4 cph[NK];
#pragma unroll
    for (int k2 = 0; k2 < NK; ++k2)
      cph[k2] = ph[k2];
    f32x4 nw = ps;
    if constexpr (REV)
      load(seg > 0 ? seg - 1 : seg);  // the last step re-reads its own maps: no branch
    else
      load(seg + 1 < G ? seg + 1 : seg);
#pragma unroll
    for (int k2 = 0; k2 < NK; ++k2)
      mm<float>(nw, cph[k2], col[k2][lane]);
    lds_barrier();  // every wave has read the column before it is overwritten
    s = nw;
  }
  if (S_final) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S_final[static_cast<size_t>(bh) * D * D + at(i)] = s[i];
  }
}

template <typename IO, int D, int C>
hipError_t launch_segmap(const chunk_args &a, float *Phi, float *Psi, hipStream_t st) {
  typedef segmap_cfg<IO, D, C> K;
  const long units_pad = (static_cast<long>(a.num_seqs) * a.H + 7) / 8 * 8;
  hipLaunchKernelGGL((gdn2_segmap_kernel<IO, D, C>), dim3(static_cast<unsigned>(units_pad * 2 * K::NSPL)),
                     dim3(64 * (K::NW + K::NL)), 0, st, a, Phi, Psi);
  return hipGetLastError();
}

template <int D>
hipError_t launch_seg_combine(const float *Phi, const float *Psi, const float *S0, int G, int H, int B,
                              float *S_in, float *S_final, hipStream_t st, bool reverse) {
  if (reverse)
    hipLaunchKernelGGL((gdn2_seg_combine_kernel<D, true>), dim3(B * H * (D / 16)), dim3(64 * (D / 16)), 0, st, Phi,
                       Psi, S0, G, H, B, S_in, S_final);
  else
    hipLaunchKernelGGL((gdn2_seg_combine_kernel<D, false>), dim3(B * H * (D / 16)), dim3(64 * (D / 16)), 0, st, Phi,
                       Psi, S0, G, H, B, S_in, S_final);
  return hipGetLastError();
}

// Bounds of G segments of each of B sequences laid end to end: sequence b
// spans [cu[b], cu[b+1]) when cu is given (packed input), else [b T, b T + T).
// Its segments hold ceil(chunks / G) chunks each, the last ones shorter or
// empty: segment g starts at start_b + min(g L_b, len_b).  seg_cu[B G] is the
// end of the last sequence.
__global__ void gdn2_seg_bounds_kernel(const int32_t *__restrict__ cu, int32_t *__restrict__ seg_cu, int G, int T,
                                       int B, int C) {
  for (int i = static_cast<int>(threadIdx.x); i <= B * G; i += static_cast<int>(blockDim.x)) {
    const int b = i < B * G ? i / G : B - 1, g = i < B * G ? i - b * G : G;
    const long start = cu ? static_cast<long>(cu[b]) : static_cast<long>(b) * T;
    const long len = cu ? static_cast<long>(cu[b + 1]) - cu[b] : static_cast<long>(T);
    const long nc = (len + C - 1) / C;
    const long L = (nc + G - 1) / G * C;
    const long x = static_cast<long>(g) * L;
    seg_cu[i] = static_cast<int32_t>(start + (x < len ? x : len));
  }
}

hipError_t launch_seg_bounds(const int32_t *cu, int32_t *seg_cu, int G, int T, int B, int C, hipStream_t st) {
  if (G < 1 || B < 1 || C < 1)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(gdn2_seg_bounds_kernel, dim3(1), dim3(256), 0, st, cu, seg_cu, G, T, B, C);
  return hipGetLastError();
}

#define GDN2_INST_SEG(IO, D, C) \
  template hipError_t launch_segmap<IO, D, C>(const chunk_args &, float *, float *, hipStream_t);

GDN2_INST_SEG(float, 16, 16)
GDN2_INST_SEG(float, 32, 16)
GDN2_INST_SEG(float, 64, 16)
GDN2_INST_SEG(float, 128, 16)
GDN2_INST_SEG(float, 16, 64)
GDN2_INST_SEG(float, 32, 64)
GDN2_INST_SEG(float, 64, 64)
GDN2_INST_SEG(float, 128, 64)
GDN2_INST_SEG(bf16_t, 16, 16)
GDN2_INST_SEG(bf16_t, 32, 16)
GDN2_INST_SEG(bf16_t, 64, 16)
GDN2_INST_SEG(bf16_t, 128, 16)
GDN2_INST_SEG(bf16_t, 16, 64)
GDN2_INST_SEG(bf16_t, 32, 64)
GDN2_INST_SEG(bf16_t, 64, 64)
GDN2_INST_SEG(bf16_t, 128, 64)

template hipError_t launch_seg_combine<16>(const float *, const float *, const float *, int, int, int, float *,
                                           float *, hipStream_t, bool);
template hipError_t launch_seg_combine<32>(const float *, const float *, const float *, int, int, int, float *,
                                           float *, hipStream_t, bool);
template hipError_t launch_seg_combine<64>(const float *, const float *, const float *, int, int, int, float *,
                                           float *, hipStream_t, bool);
template hipError_t launch_seg_combine<128>(const float *, const float *, const float *, int, int, int, float *,
                                           float *, hipStream_t, bool);

}  // namespace gdn2
