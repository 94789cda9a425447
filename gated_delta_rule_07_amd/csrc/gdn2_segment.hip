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

// One workgroup per (segment, head) and map: part 0 computes Psi, part 1 Phi.
// One wave per 16-column tile of the map.  Per chunk, the workgroup lays the
// chunk's -W and Kbar^T tiles (as the prep stores them) into LDS, loaded one
// chunk ahead, and every wave takes
//   Z = [Ut] - W S,   S <- Diag(gamma_C) S + Kbar^T Z
// on its columns (Ut only for Psi).
template <typename IO, int D, int C>
__global__ void __launch_bounds__(64 * (D / 16)) gdn2_segmap_kernel(chunk_args a, float *Phi, float *Psi) {
  constexpr int NB = C / 16, NK = D / 16, NW = NK, NT2 = 2 * NB * NK;
  typedef frag<IO> F;
  typedef blk_layout<IO, D, C> L;
  constexpr size_t TB = F::TILE_BYTES;
  // [0, NB*NK): RowFrag(-W) tiles (tt, kk); [NB*NK, NT2): RowFrag(Kbar^T) tiles (kk, tt); gamma_C
  __shared__ __attribute__((aligned(16))) unsigned char sm[NT2 * TB + D * sizeof(float)];
  float *gam = reinterpret_cast<float *>(sm + NT2 * TB);

  const int unit = static_cast<int>(blockIdx.x >> 1), part = static_cast<int>(blockIdx.x & 1);
  if (unit >= a.num_seqs * a.H)
    return;
  const int n = unit / a.H, h = unit - n * a.H;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  const int j = wave;  // column tile of the map
  int c_begin, nchunks;
  if (a.cu) {
    c_begin = a.offsets[n];
    nchunks = a.offsets[n + 1] - c_begin;
  } else {
    const int nc = (a.T + C - 1) / C;
    c_begin = n * nc;
    nchunks = nc;
  }
  f32x4 s[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s[kk][i] = (part == 1 && kk == j && 4 * g + i == m) ? 1.f : 0.f;

  constexpr int PPW = (NT2 + NW - 1) / NW;
  F raw[PPW], utn[NB], ut[NB];
  float gamv = 0.f;
  auto issue = [&](int c) {
    const unsigned char *blk =
        reinterpret_cast<const unsigned char *>(a.blocks) + (static_cast<size_t>(c_begin + c) * a.H + h) * a.blk_bytes;
#pragma unroll
    for (int r = 0; r < PPW; ++r) {
      const int p = wave + r * NW;
      if (p < NT2) {
        if (p < NB * NK) {
          const int tt = p / NK, kk = p - tt * NK;
          raw[r] = F::ld_at(blk + L::WN + tile_off<IO, NK>(tt, kk, lane));
        } else {
          const int q2 = p - NB * NK, kk = q2 / NB, tt = q2 - kk * NB;
          raw[r] = F::ld_at(blk + L::KB + tile_off<IO, NB>(kk, tt, lane));
        }
      }
    }
    if (threadIdx.x < D)
      gamv = reinterpret_cast<const float *>(blk + L::GAM)[threadIdx.x];
    if (part == 0) {
#pragma unroll
      for (int tt = 0; tt < NB; ++tt)
        utn[tt] = F::ld_at(blk + L::UT + tile_off<IO, NK>(tt, j, lane));
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int r = 0; r < PPW; ++r) {
      const int p = wave + r * NW;
      if (p < NT2)
        raw[r].st(sm + static_cast<size_t>(p) * TB, lane);
    }
    if (threadIdx.x < D)
      gam[threadIdx.x] = gamv;
#pragma unroll
    for (int tt = 0; tt < NB; ++tt)
      ut[tt] = utn[tt];
  };
  if (nchunks > 0) {
    issue(0);
    commit();
  }
  lds_barrier();
  for (int c = 0; c < nchunks; ++c) {
    issue(c + 1 < nchunks ? c + 1 : c);  // the last step re-reads its own chunk: no branch
    F sf[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      sf[kk] = F::from(s[kk]);
    F zf[NB];
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
      f32x4 z = (part == 0) ? ut[tt].to_f32() : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        mm_io(z, F::ld(sm + static_cast<size_t>(tt * NK + kk) * TB, lane), sf[kk]);
      zf[tt] = F::from(z);
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      s[kk] *= *reinterpret_cast<const f32x4 *>(gam + 16 * kk + 4 * g);
#pragma unroll
      for (int tt = 0; tt < NB; ++tt)
        mm_io(s[kk], F::ld(sm + static_cast<size_t>(NB * NK + kk * NB + tt) * TB, lane), zf[tt]);
    }
    lds_barrier();  // this chunk's tiles are no longer read
    if (c + 1 < nchunks)
      commit();
    lds_barrier();
  }
  float *out = (part == 0 ? Psi : Phi) + static_cast<size_t>(unit) * D * D;
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out[(16 * kk + 4 * g + i) * D + 16 * j + m] = s[kk][i];
}

// One wave per (head, 16-column tile of the state).  Segments g = 0 .. G-1
// of one sequence, maps [G][H][D][D]: writes the state entering every
// segment to S_in [G][H][D][D] and, if S_final is given, the state after
// the last one.  float32 throughout (products as in mm<float>).
template <int D>
__global__ void __launch_bounds__(64) gdn2_seg_combine_kernel(const float *__restrict__ Phi,
                                                              const float *__restrict__ Psi,
                                                              const float *__restrict__ S0, int G, int H,
                                                              float *__restrict__ S_in, float *__restrict__ S_final) {
  constexpr int NK = D / 16;
  const int h = static_cast<int>(blockIdx.x) / NK, j = static_cast<int>(blockIdx.x) % NK;
  if (h >= H)
    return;
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  auto at = [&](int kk, int i) { return static_cast<size_t>(16 * kk + 4 * g + i) * D + 16 * j + m; };
  f32x4 s[NK];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      s[kk][i] = S0 ? S0[static_cast<size_t>(h) * D * D + at(kk, i)] : 0.f;
  for (int seg = 0; seg < G; ++seg) {
    const size_t base = (static_cast<size_t>(seg) * H + h) * D * D;
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S_in[base + at(kk, i)] = s[kk][i];
    if (seg + 1 == G && !S_final)
      break;
    f32x4 nw[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        nw[kk][i] = Psi[base + at(kk, i)];
#pragma unroll
      for (int k2 = 0; k2 < NK; ++k2) {
        // RowFrag(Phi tile (kk, k2)): row 16 kk + m, columns 16 k2 + 4 g .. +3
        const f32x4 ph = *reinterpret_cast<const f32x4 *>(Phi + base + static_cast<size_t>(16 * kk + m) * D + 16 * k2 + 4 * g);
        mm<float>(nw[kk], ph, s[k2]);
      }
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
      s[kk] = nw[kk];
  }
  if (S_final) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S_final[static_cast<size_t>(h) * D * D + at(kk, i)] = s[kk][i];
  }
}

template <typename IO, int D, int C>
hipError_t launch_segmap(const chunk_args &a, float *Phi, float *Psi, hipStream_t st) {
  const int units = a.num_seqs * a.H;
  hipLaunchKernelGGL((gdn2_segmap_kernel<IO, D, C>), dim3(2 * units), dim3(64 * (D / 16)), 0, st, a, Phi, Psi);
  return hipGetLastError();
}

template <int D>
hipError_t launch_seg_combine(const float *Phi, const float *Psi, const float *S0, int G, int H, float *S_in,
                              float *S_final, hipStream_t st) {
  hipLaunchKernelGGL((gdn2_seg_combine_kernel<D>), dim3(H * (D / 16)), dim3(64), 0, st, Phi, Psi, S0, G, H, S_in,
                     S_final);
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

template hipError_t launch_seg_combine<16>(const float *, const float *, const float *, int, int, float *, float *,
                                           hipStream_t);
template hipError_t launch_seg_combine<32>(const float *, const float *, const float *, int, int, float *, float *,
                                           hipStream_t);
template hipError_t launch_seg_combine<64>(const float *, const float *, const float *, int, int, float *, float *,
                                           hipStream_t);
template hipError_t launch_seg_combine<128>(const float *, const float *, const float *, int, int, float *, float *,
                                            hipStream_t);

}  // namespace gdn2
