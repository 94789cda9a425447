// gdn2_fused.hip -- single-pass chunkwise GDN-2 forward for gfx950.
//
// One workgroup of C/16 waves owns one (sequence, head) -- or one of NG
// column groups of it -- and walks its chunks in order.  For each chunk it
// runs the per-chunk phases of gdn2_wy.hpp (decay prefix sums, gated
// operands, A and P, T = (I + A)^{-1}, W, Q', Ut, O_intra) with every
// intermediate in LDS or registers, then advances the state held in
// matrix-core accumulators:
//   Z = Ut - W S,  O = O_intra + Q' S  (written to o),  S <- Diag(gamma_C) S + Kbar^T Z.
// HBM traffic is the inputs once, the outputs once and the states: no
// workspace round trip.  The next chunk's inputs are loaded into registers as
// soon as the current chunk's have been consumed, so their latency overlaps
// the matrix phases and the state step.
//
// Column groups (NG > 1) split dv between workgroups of the same head; each
// of them recomputes the dk-side phases, which trades duplicate work for
// twice as many workgroups when there are fewer heads than compute units.
#include "gdn2_wy.hpp"

namespace gdn2 {

template <typename IO, int D, int C, int NG> struct fused_cfg {
  static constexpr int NB = C / 16, NK = D / 16;
  static constexpr int CTK = NK / NB;         // dk tiles of W, Q' per wave
  static constexpr int NVW = NK / (NG * NB);  // dv tiles (state columns) per wave
  static constexpr size_t LDS = sizeof(wy_smem<IO, D, C>) + blk_layout<IO, D, C>::SHARED0;
  static constexpr bool OK = NK % NB == 0 && NK % (NG * NB) == 0 && NVW >= 1 && LDS <= 160 * 1024;
};

// grid: units_pad * NG workgroups (units_pad = N*H rounded up to 8; all
// column groups of a head share an XCD); block: 64 * C/16 threads.
template <typename IO, int D, int C, int NG, int GM>
__global__ void __launch_bounds__(64 * (C / 16)) gdn2_fused_kernel(chunk_args a) {
  typedef fused_cfg<IO, D, C, NG> K;
  constexpr int NB = K::NB, NK = K::NK, CTK = K::CTK, NVW = K::NVW;
  typedef frag<IO> F;
  typedef frag2<IO> F2;
  typedef blk_layout<IO, D, C> L;
  __shared__ wy_smem<IO, D, C> sm;
  // -W, Q', Kbar^T and gamma_C of the current chunk, in the block layout
  __shared__ __attribute__((aligned(16))) unsigned char tiles[L::SHARED0];

  const int x = blockIdx.x;
  const int xcd = x & 7, s8 = x >> 3;
  const int unit = (s8 / NG) * 8 + xcd;
  const int cg = s8 % NG;
  if (unit >= a.num_seqs * a.H)
    return;
  const int n = unit / a.H, h = unit - n * a.H;
  const int tid = threadIdx.x;
  const int I = tid >> 6, lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int vt0 = cg * (NK / NG) + I * NVW;  // first state column tile of this wave
  int c_begin, nchunks;
  long tstart, tend;
  sequence_range<C>(n, a, c_begin, nchunks, tstart, tend);
  (void)c_begin;

  f32x4 S[NK][NVW];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int j = 0; j < NVW; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[kk][j][i] = a.S0 ? a.S0[(static_cast<size_t>(unit) * D + 16 * kk + 4 * g + i) * D +
                                  16 * (vt0 + j) + m]
                           : 0.f;
  IO *out = static_cast<IO *>(a.o);
  const F eye = identity_colfrag<IO>(lane);

  constexpr bool LP = GM == GM_LAYER;
  wy_rows<IO, D, LP> r;
  raw4<IO> rv[NB][NVW], rw[NB][NVW];
  if (nchunks > 0) {
    const int len0 = (tend - tstart) < C ? static_cast<int>(tend - tstart) : C;
    wy_load_chunk<IO, D, C, NVW, GM>(a, tstart, len0, h, I, vt0, true, m, g, r, rv, rw);
  }
  // outputs of the previous chunk, stored once this chunk's inputs have been
  // consumed (so that waiting for the prefetched inputs never waits for them)
  f32x4 po[NVW][NB];
  long pt0 = 0;
  int plen = 0;
  auto store_prev = [&]() {
#pragma unroll
    for (int j = 0; j < NVW; ++j)
#pragma unroll
      for (int tt = 0; tt < NB; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * tt + 4 * g + i;
          if (t < plen)
            out[(static_cast<size_t>(pt0 + t) * a.H + h) * D + 16 * (vt0 + j) + m] = io<IO>::from_f(po[j][tt][i]);
        }
  };
  for (int c = 0; c < nchunks; ++c) {
    const long t0 = tstart + static_cast<long>(c) * C;
    const int len = (tend - t0) < C ? static_cast<int>(tend - t0) : C;

    f32x4 gl[NK];
    bool pw;
    wy_decay<IO, D, C, LP>(sm, r, gl, pw, a, t0, len, h, I, tid, reinterpret_cast<float *>(tiles + L::GAM));
    wy_ops<IO, D> op;
    wy_operands<IO, D, C, LP>(sm, r, gl, pw, a, t0, len, h, I, lane, eye, tiles + L::KB, op);
    F ucol[NB][NVW];
    wy_values<IO, NB, NVW, LP>(rv, rw, eye, ucol);
    if (c > 0)
      store_prev();
    if (c + 1 < nchunks) {  // inputs of the next chunk, while this one computes
      const long tn = t0 + C;
      const int lenn = (tend - tn) < C ? static_cast<int>(tend - tn) : C;
      wy_load_chunk<IO, D, C, NVW, GM>(a, tn, lenn, h, I, vt0, true, m, g, r, rv, rw);
    }
    __syncthreads();
    F af[NB];
    wy_products<IO, D, C>(sm, op, I, lane, af);
    wy_inverse<IO, D, C>(sm, af, I, lane, eye);
    wy_tp<IO, C> tp;
    wy_load_tp<IO, D, C>(sm, lane, tp);
#pragma unroll
    for (int j = 0; j < CTK; ++j)
      wy_wq<IO, D, C>(sm, tp, I * CTK + j, lane, eye, tiles + L::WN, tiles + L::QP);
    f32x4 ut[NVW][NB], oi[NVW][NB];
#pragma unroll
    for (int j = 0; j < NVW; ++j) {
      F uc_j[NB];
#pragma unroll
      for (int J = 0; J < NB; ++J)
        uc_j[J] = ucol[J][j];
      wy_uo<IO, C>(tp, uc_j, ut[j], oi[j]);
    }
    __syncthreads();  // -W, Q', Kbar^T, gamma of this chunk are complete

    // ---- state step for this wave's column tiles; operand tiles are loaded
    // once and shared by the wave's column tiles
    F sf[NVW][NK];
#pragma unroll
    for (int j = 0; j < NVW; ++j)
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
        sf[j][kk] = F::from(S[kk][j]);
    F zf[NVW][NB];
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
      if constexpr (NK % 2 == 0) {
        F2 wa[NK / 2], qa[NK / 2];
#pragma unroll
        for (int k2 = 0; k2 < NK / 2; ++k2) {
          wa[k2] = F2::ld(tiles + L::WN + tile_off<IO, NK>(tt, 2 * k2, 0), lane);
          qa[k2] = F2::ld(tiles + L::QP + tile_off<IO, NK>(tt, 2 * k2, 0), lane);
        }
#pragma unroll
        for (int j = 0; j < NVW; ++j) {
          // ut / oi come out of 16x16x16 products: they are added on the
          // vector ALU rather than used as the accumulator of the 16x16x32
          // chain (see mma32)
          f32x4 z = {0.f, 0.f, 0.f, 0.f};
          f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int k2 = 0; k2 < NK / 2; ++k2) {
            const F2 sb2 = F2::make(sf[j][2 * k2], sf[j][2 * k2 + 1]);
            mma32(z, wa[k2], sb2);
            mma32(o, qa[k2], sb2);
          }
          z += ut[j][tt];
          o += oi[j][tt];
          zf[j][tt] = F::from(z);
          po[j][tt] = o;
        }
      } else {
        F wa[NK], qa[NK];
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          wa[kk] = F::ld(tiles + L::WN + tile_off<IO, NK>(tt, kk, 0), lane);
          qa[kk] = F::ld(tiles + L::QP + tile_off<IO, NK>(tt, kk, 0), lane);
        }
#pragma unroll
        for (int j = 0; j < NVW; ++j) {
          f32x4 z = ut[j][tt];
          f32x4 o = oi[j][tt];
#pragma unroll
          for (int kk = 0; kk < NK; ++kk) {
            mma16(z, wa[kk], sf[j][kk]);
            mma16(o, qa[kk], sf[j][kk]);
          }
          zf[j][tt] = F::from(z);
          po[j][tt] = o;
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const f32x4 gam = *reinterpret_cast<const f32x4 *>(tiles + L::GAM + (16 * kk + 4 * g) * sizeof(float));
      if constexpr (NB % 2 == 0) {
        F2 ka[NB / 2];
#pragma unroll
        for (int t2 = 0; t2 < NB / 2; ++t2)
          ka[t2] = F2::ld(tiles + L::KB + tile_off<IO, NB>(kk, 2 * t2, 0), lane);
#pragma unroll
        for (int j = 0; j < NVW; ++j) {
          S[kk][j] *= gam;
#pragma unroll
          for (int t2 = 0; t2 < NB / 2; ++t2)
            mma32(S[kk][j], ka[t2], F2::make(zf[j][2 * t2], zf[j][2 * t2 + 1]));
        }
      } else {
        F ka[NB];
#pragma unroll
        for (int tt = 0; tt < NB; ++tt)
          ka[tt] = F::ld(tiles + L::KB + tile_off<IO, NB>(kk, tt, 0), lane);
#pragma unroll
        for (int j = 0; j < NVW; ++j) {
          S[kk][j] *= gam;
#pragma unroll
          for (int tt = 0; tt < NB; ++tt)
            mma16(S[kk][j], ka[tt], zf[j][tt]);
        }
      }
    }
    pt0 = t0;
    plen = len;
  }
  if (nchunks > 0)
    store_prev();
  if (a.S_final) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int j = 0; j < NVW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.S_final[(static_cast<size_t>(unit) * D + 16 * kk + 4 * g + i) * D + 16 * (vt0 + j) + m] =
              S[kk][j][i];
  }
}

template <typename IO, int D, int C, int NG> bool fused_supported() { return fused_cfg<IO, D, C, NG>::OK; }

template <typename IO, int D, int C, int NG> hipError_t launch_fused(const chunk_args &a, hipStream_t st) {
  if constexpr (fused_cfg<IO, D, C, NG>::OK) {
    const int units = a.num_seqs * a.H;
    const int units_pad = (units + 7) / 8 * 8;
    const dim3 grid(units_pad * NG), block(64 * (C / 16));
    const uint32_t kda = GATE_SCALAR_B | GATE_SCALAR_W;
    if (a.gates & GATE_LAYER_PREP)
      hipLaunchKernelGGL((gdn2_fused_kernel<IO, D, C, NG, GM_LAYER>), grid, block, 0, st, a);
    else if (a.gates == kda)
      hipLaunchKernelGGL((gdn2_fused_kernel<IO, D, C, NG, GM_KDA>), grid, block, 0, st, a);
    else if (a.gates == (kda | GATE_SCALAR_ALPHA))
      hipLaunchKernelGGL((gdn2_fused_kernel<IO, D, C, NG, GM_GDN>), grid, block, 0, st, a);
    else if (a.gates)
      hipLaunchKernelGGL((gdn2_fused_kernel<IO, D, C, NG, GM_GATES>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((gdn2_fused_kernel<IO, D, C, NG, GM_PLAIN>), grid, block, 0, st, a);
    return hipGetLastError();
  } else {
    return hipErrorInvalidConfiguration;
  }
}

#define GDN2_INST_FUSED(IO, D, C, NG)                                                 \
  template bool fused_supported<IO, D, C, NG>();                                    \
  template hipError_t launch_fused<IO, D, C, NG>(const chunk_args &, hipStream_t);

// every size gets a symbol; sizes without a kernel (fused_cfg::OK false)
// report it and refuse to launch
GDN2_INST_FUSED(float, 16, 16, 1)
GDN2_INST_FUSED(float, 16, 16, 2)
GDN2_INST_FUSED(float, 16, 64, 1)
GDN2_INST_FUSED(float, 16, 64, 2)
GDN2_INST_FUSED(float, 32, 16, 1)
GDN2_INST_FUSED(float, 32, 16, 2)
GDN2_INST_FUSED(float, 32, 64, 1)
GDN2_INST_FUSED(float, 32, 64, 2)
GDN2_INST_FUSED(float, 64, 16, 1)
GDN2_INST_FUSED(float, 64, 16, 2)
GDN2_INST_FUSED(float, 64, 64, 1)
GDN2_INST_FUSED(float, 64, 64, 2)
GDN2_INST_FUSED(float, 128, 16, 1)
GDN2_INST_FUSED(float, 128, 16, 2)
GDN2_INST_FUSED(float, 128, 64, 1)
GDN2_INST_FUSED(float, 128, 64, 2)
GDN2_INST_FUSED(bf16_t, 16, 16, 1)
GDN2_INST_FUSED(bf16_t, 16, 16, 2)
GDN2_INST_FUSED(bf16_t, 16, 64, 1)
GDN2_INST_FUSED(bf16_t, 16, 64, 2)
GDN2_INST_FUSED(bf16_t, 32, 16, 1)
GDN2_INST_FUSED(bf16_t, 32, 16, 2)
GDN2_INST_FUSED(bf16_t, 32, 64, 1)
GDN2_INST_FUSED(bf16_t, 32, 64, 2)
GDN2_INST_FUSED(bf16_t, 64, 16, 1)
GDN2_INST_FUSED(bf16_t, 64, 16, 2)
GDN2_INST_FUSED(bf16_t, 64, 64, 1)
GDN2_INST_FUSED(bf16_t, 64, 64, 2)
GDN2_INST_FUSED(bf16_t, 128, 16, 1)
GDN2_INST_FUSED(bf16_t, 128, 16, 2)
GDN2_INST_FUSED(bf16_t, 128, 64, 1)
GDN2_INST_FUSED(bf16_t, 128, 64, 2)

}  // namespace gdn2
