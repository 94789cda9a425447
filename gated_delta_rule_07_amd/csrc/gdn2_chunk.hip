// gdn2_chunk.hip -- two-pass chunkwise GDN-2 forward for gfx950.
//
// Pass 1 (gdn2_chunk_prep_kernel) runs the per-chunk phases of gdn2_wy.hpp for
// every (chunk, head) in parallel and writes the chunk's -W, Q', Kbar^T,
// gamma_C, Ut and O_intra to the workspace in fragment order.  Pass 2
// (gdn2_chunk_scan_kernel) walks the chunks of each sequence in order with
// the state in matrix-core accumulators.  This path keeps the whole GPU busy
// when there are few (sequence, head) units (long sequences, small batch);
// gdn2_fused.hip does both passes in one workgroup per head and avoids the
// workspace round trip when there are enough units.  gdn2_chunk_table_kernel
// builds the per-sequence chunk offsets of packed input.
#include "gdn2_wy.hpp"

namespace gdn2 {

template <typename IO, int D, int C> size_t chunk_block_bytes() { return blk_layout<IO, D, C>::BYTES; }

// Pass 1.  grid: num_slots * H, block: 64 * C/16 threads (see gdn2_wy.hpp for
// the work split between waves).
template <typename IO, int D, int C>
__global__ void __launch_bounds__(64 * (C / 16)) gdn2_chunk_prep_kernel(chunk_args a) {
  constexpr int NB = C / 16, NK = D / 16;
  constexpr int CTW = (NK >= NB) ? NK / NB : 1;  // column tiles per wave
  typedef frag<IO> F;
  typedef blk_layout<IO, D, C> L;
  __shared__ wy_smem<IO, D, C> sm;

  const int h = blockIdx.x % a.H;
  const int slot = blockIdx.x / a.H;
  int seq, len;
  long t0;
  if (!locate_chunk<C>(slot, a, seq, t0, len))
    return;  // whole workgroup leaves together
  (void)seq;
  const int tid = threadIdx.x;
  const int I = tid >> 6;
  const int lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int ct0 = I * CTW;
  const bool owner = ct0 < NK;
  unsigned char *blk = reinterpret_cast<unsigned char *>(a.blocks) +
                       (static_cast<size_t>(slot) * a.H + h) * a.blk_bytes;

  wy_rows<IO, D> r;
  wy_load_rows<IO, D>(a, t0, len, h, 16 * I + m, g, r);
  raw4<IO> rv[NB][CTW], rw[NB][CTW];
  wy_load_vw<IO, D, C, CTW>(a, t0, len, h, ct0, owner, m, g, rv, rw);
  f32x4 gl[NK];
  wy_decay<IO, D, C>(sm, r, gl, I, tid, reinterpret_cast<float *>(blk + L::GAM));
  const F eye = identity_colfrag<IO>(lane);
  wy_ops<IO, D> op;
  wy_operands<IO, D, C>(sm, r, gl, I, lane, eye, blk + L::KB, op);
  F ucol[NB][CTW];
  wy_values<IO, NB, CTW>(rv, rw, eye, ucol);
  __syncthreads();
  F af[NB];
  wy_products<IO, D, C>(sm, op, I, lane, af);
  wy_inverse<IO, D, C>(sm, af, I, lane, eye);
  if (owner) {
    wy_tp<IO, C> tp;
    wy_load_tp<IO, D, C>(sm, lane, tp);
#pragma unroll
    for (int j = 0; j < CTW; ++j) {
      const int ct = ct0 + j;
      wy_wq<IO, D, C>(sm, tp, ct, lane, eye, blk + L::WN, blk + L::QP);
      F uc_j[NB];
#pragma unroll
      for (int J = 0; J < NB; ++J)
        uc_j[J] = ucol[J][j];
      f32x4 ut[NB], oi[NB];
      wy_uo<IO, C>(tp, uc_j, ut, oi);
#pragma unroll
      for (int I2 = 0; I2 < NB; ++I2) {
        F::from(ut[I2]).st(blk + L::UT + (I2 * NK + ct) * L::TB, lane);
        F::from(oi[I2]).st(blk + L::OI + (I2 * NK + ct) * L::TB, lane);
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
