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

// Per chunk every compute wave takes
//   Z = [Ut] - W S,   S <- Diag(gamma_C) S + Kbar^T Z
// on its CPW 16-column tiles of one map (Ut only for Psi; Phi starts from
// the identity) from the chunk's -W and Kbar^T tiles, its Ut tiles and
// gamma_C, staged in LDS: the -W and Kbar^T regions of the prep's block are
// copied byte for byte (16 or 8 bytes a lane), so they keep the block's
// tile order, with 16-wide k tiles paired; bfloat16 products then take two
// k tiles per 16x16x32 instruction.
// bfloat16 (MERGED): NSPL = NK / CPW workgroups per (segment, head), each
// with two compute waves on the same CPW = 2 column tiles, wave 0 of Psi
// and wave 1 of Phi, so both maps share one staged copy of each chunk and
// every -W and Kbar^T fragment read from LDS serves two column tiles; NL
// loader waves stage the chunks into two LDS buffers, chunk k by loader
// (k - 1) mod NL, which issues its loads NL chunks before they are due, so
// the compute waves never wait on global memory (one barrier per chunk).
// float32: two workgroups per (segment, head), part 0 of Psi and part 1 of
// Phi, each with one compute wave per column tile, which stage the tiles
// themselves one chunk ahead (loader registers would not hold float32
// chunks).  Every workgroup of one (segment, head) sits on the same XCD,
// whose L2 serves their common reads.
// Grid: units_pad * NPART * NSPL workgroups, units_pad = N*H rounded up to 8.
// CW: column tiles per compute wave when merged (1 or 2; 2 needs NK even),
// chosen at launch: two halve the workgroups, which pays once there are
// enough of them to fill the compute units.
template <typename IO, int D, int C, int CW> struct segmap_cfg {
  static constexpr int NK = D / 16, NB = C / 16;
  static constexpr bool PIPE = sizeof(IO) == 2;
  static constexpr bool MERGED = PIPE;                              // both maps in one workgroup
  static constexpr int CPW = (MERGED && NK % 2 == 0 && CW == 2) ? 2 : 1;  // column tiles per compute wave
  // staged Ut bytes per row tile (merged): the stored pair holding the
  // wave's tiles, or the one tile when NK is odd (no pairs)
  static constexpr size_t UTS = (NK % 2 == 0 ? 2 : 1) * frag<IO>::TILE_BYTES;
  static constexpr int NSPL = MERGED ? NK / CPW : 1;            // workgroups per (segment, head) and part
  static constexpr int NPART = MERGED ? 1 : 2;                  // parts (maps) in the grid
  static constexpr int NW = MERGED ? 2 : NK;                    // compute waves
  static constexpr int NL = PIPE ? 2 : 0;
  static constexpr int NBUF = PIPE ? 2 : 1;
  static constexpr size_t TB = frag<IO>::TILE_BYTES;
  static constexpr size_t RB = static_cast<size_t>(NB) * NK * TB;  // bytes of the -W region, and of Kbar^T's
  static constexpr int PW = RB % 1024 == 0 ? 16 : 8;                // bytes a lane copies per piece
  static constexpr size_t PB = 64 * PW;                              // bytes of one piece
  static constexpr int NRP = static_cast<int>(2 * RB / PB);          // pieces of the two regions
  static constexpr int NUT = NW * NB;                               // staged Ut tiles (not merged)
  static constexpr size_t UTO = 2 * RB, GMO = 2 * RB + (MERGED ? NB * UTS : NUT * TB);  // Ut tiles, gamma_C
  static constexpr size_t BUF = GMO + D * sizeof(float);
};

template <typename IO, int D, int C, int CW>
__global__ void __launch_bounds__((64 * (segmap_cfg<IO, D, C, CW>::NW + segmap_cfg<IO, D, C, CW>::NL)))
    gdn2_segmap_kernel(chunk_args a, float *Phi, float *Psi) {
  typedef segmap_cfg<IO, D, C, CW> K;
  constexpr int NB = C / 16, NK = D / 16, NW = K::NW, NSPL = K::NSPL, NL = K::NL, NRP = K::NRP, CPW = K::CPW,
                NPART = K::NPART, NUT = K::NUT;
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
  const int unit = (s8 / (NPART * NSPL)) * 8 + xcd;
  const int gpart = (s8 % (NPART * NSPL)) / NSPL, grp = s8 % NSPL;
  if (unit >= a.num_seqs * a.H)
    return;  // whole workgroup
  const int n = unit / a.H, h = unit - n * a.H;
  if (a.seg_G > 0 && n % a.seg_G == a.seg_G - 1)
    return;  // whole workgroup: the last segment's map is not needed
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
  // this lane's fragment of staged Ut tile i (column tile i / NB of the
  // workgroup, row tile i % NB), in the block
  auto ut_src = [&](int i) -> size_t {
    const int col = K::MERGED ? CPW * grp + i / NB : grp * NW + i / NB;
    return L::UT + tile_off<IO, NK>(i % NB, col, lane);
  };

  if constexpr (NL > 0) {
    if (wave >= NW) {
      // ---- loader wave (bfloat16, MERGED): chunk c + 1 is copied into LDS
      // buffer (c + 1) % 2 by loader (c + 1) mod NL while the compute waves
      // take chunk c, with direct global -> LDS loads (16 bytes a lane; 4
      // for a tail under 1 KB): the block's -W and Kbar^T regions byte for
      // byte, the workgroup's Ut tiles of each row tile (one stored pair,
      // or one tile when NK is odd), and gamma_C.  No registers hold the
      // data, and the copy is waited for (vmcnt) before the barrier that
      // hands the buffer over.
      if (nchunks == 0)
        return;  // no barrier is taken
      const int l = wave - NW;
      auto dma = [&](const unsigned char *src, unsigned char *dst, int n) {
        int o = 0;
        for (; o + 1024 <= n; o += 1024)
          __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(src + o + 16 * lane),
                                           (__attribute__((address_space(3))) void *)(dst + o), 16, 0, 0);
        for (; o < n; o += 256)
          if (o + 4 * lane < n)
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)(src + o + 4 * lane),
                                             (__attribute__((address_space(3))) void *)(dst + o), 4, 0, 0);
      };
      auto stage = [&](int c, int bsel) {
        const unsigned char *blk = blk_of(c);
        unsigned char *dst = &sbuf[bsel][0];
        dma(blk + L::WN, dst, static_cast<int>(RB));
        dma(blk + L::KB, dst + RB, static_cast<int>(RB));
        const int ucol = NK % 2 == 0 ? (CPW * grp) & ~1 : grp;  // first column tile of the staged Ut
#pragma unroll
        for (int tt = 0; tt < NB; ++tt)
          dma(blk + L::UT + tile_off<IO, NK>(tt, ucol, 0), dst + K::UTO + static_cast<size_t>(tt) * K::UTS,
              static_cast<int>(K::UTS));
        dma(blk + L::GAM, dst + K::GMO, static_cast<int>(D * sizeof(float)));
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      };
      if (l == 0)
        stage(0, 0);
      lds_barrier();  // chunk 0 is staged
      for (int i = 0; i < nchunks; ++i) {
        if (i + 1 < nchunks && (i + 1) % NL == l)
          stage(i + 1, (i + 1) % 2);  // buffer (i + 1) % 2 was freed by the previous barrier
        lds_barrier();  // chunk i + 1 is staged, chunk i's buffer is free
      }
      return;
    }
  }

  // ---- compute wave: column tiles jb .. jb + CPW - 1 of one map
  const int part = K::MERGED ? wave : gpart;  // 0: Psi, 1: Phi
  const int jb = K::MERGED ? CPW * grp : grp * NW + wave;
  const int ub = K::MERGED ? 0 : wave * NB;  // first staged Ut tile of this wave
  f32x4 s[NK][CPW];
#pragma unroll
  for (int kk = 0; kk < NK; ++kk)
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s[kk][c][i] = (part == 1 && kk == jb + c && 4 * g + i == m) ? 1.f : 0.f;

  // the products of one chunk from its staged buffer (each -W and Kbar^T
  // fragment read once for the wave's CPW column tiles)
  constexpr bool PAIR_K = sizeof(IO) == 2 && NK % 2 == 0, PAIR_T = sizeof(IO) == 2 && NB % 2 == 0;
  auto step = [&](const unsigned char *sb) {
    F sf[NK][CPW];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int c = 0; c < CPW; ++c)
        sf[kk][c] = F::from(s[kk][c]);
    F zf[NB][CPW];
#pragma unroll
    for (int tt = 0; tt < NB; ++tt) {
      f32x4 z[CPW];
      if (part != 0) {
#pragma unroll
        for (int c = 0; c < CPW; ++c)
          z[c] = f32x4{0.f, 0.f, 0.f, 0.f};
      } else if constexpr (K::MERGED && NK % 2 == 0) {
        const F2 u2 = F2::ld(sb + K::UTO + static_cast<size_t>(tt) * K::UTS, lane);  // row tile tt's stored pair
        if constexpr (CPW == 2) {
          z[0] = u2.lo.to_f32();
          z[1] = u2.hi.to_f32();
        } else {
          z[0] = ((grp & 1) ? u2.hi : u2.lo).to_f32();
        }
      } else {
#pragma unroll
        for (int c = 0; c < CPW; ++c)
          z[c] = F::ld(sb + K::UTO + (K::MERGED ? static_cast<size_t>(tt) : static_cast<size_t>(ub + tt)) * TB,
                       lane).to_f32();
      }
      if constexpr (PAIR_K) {
#pragma unroll
        for (int kp = 0; kp < NK / 2; ++kp) {
          const F2 w2 = F2::ld(sb + tile_off<IO, NK>(tt, 2 * kp, 0), lane);
#pragma unroll
          for (int c = 0; c < CPW; ++c)
            mma32(z[c], w2, F2::make(sf[2 * kp][c], sf[2 * kp + 1][c]));
        }
      } else {
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const F w1 = F::ld_at(sb + tile_off<IO, NK>(tt, kk, lane));
#pragma unroll
          for (int c = 0; c < CPW; ++c)
            mm_io(z[c], w1, sf[kk][c]);
        }
      }
#pragma unroll
      for (int c = 0; c < CPW; ++c)
        zf[tt][c] = F::from(z[c]);
    }
    const float *gam = reinterpret_cast<const float *>(sb + K::GMO);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const f32x4 gm = *reinterpret_cast<const f32x4 *>(gam + 16 * kk + 4 * g);
#pragma unroll
      for (int c = 0; c < CPW; ++c)
        s[kk][c] *= gm;
      if constexpr (PAIR_T) {
#pragma unroll
        for (int tp = 0; tp < NB / 2; ++tp) {
          const F2 kb = F2::ld(sb + RB + tile_off<IO, NB>(kk, 2 * tp, 0), lane);
#pragma unroll
          for (int c = 0; c < CPW; ++c)
            mma32(s[kk][c], kb, F2::make(zf[2 * tp][c], zf[2 * tp + 1][c]));
        }
      } else {
#pragma unroll
        for (int tt = 0; tt < NB; ++tt) {
          const F kb = F::ld_at(sb + RB + tile_off<IO, NB>(kk, tt, lane));
#pragma unroll
          for (int c = 0; c < CPW; ++c)
            mm_io(s[kk][c], kb, zf[tt][c]);
        }
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
          u[tt] = F::ld_at(blk + ut_src(wave * NB + tt));
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
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[(16 * kk + 4 * g + i) * D + 16 * (jb + c) + m] = s[kk][c][i];
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
// GC > 0: the segment count is GC (G is ignored) and the step loop is
// unrolled whole, so that the maps loaded two steps ahead land in fresh
// registers; with a run-time count the loop carries them in fixed registers
// and each step waits for the loads it has just issued.
template <int D, bool REV = false, int GC = 0>
__global__ void __launch_bounds__(64 * (D / 16)) gdn2_seg_combine_kernel(const float *__restrict__ Phi,
                                                                         const float *__restrict__ Psi,
                                                                         const float *__restrict__ S0, int G_rt, int H,
                                                                         int B, float *__restrict__ S_in,
                                                                         float *__restrict__ S_final) {
  constexpr int NK = D / 16;
  const int G = GC > 0 ? GC : G_rt;
  __shared__ f32x4 col[NK][64];  // ColFrag of the state tiles (k2, j)
  // consecutive workgroup ids go to the 8 XCDs in turn; the NK column tiles
  // of one (sequence, head) all take ids of one XCD, whose L2 then serves
  // their common reads of every Phi (grid: (B H rounded up to 8) x NK)
  const int x = static_cast<int>(blockIdx.x), r = x >> 3;
  const int bh = (r / NK) * 8 + (x & 7), j = r % NK;
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
  // two sets of RowFrag(Phi) (REV: Phi^T) tiles (kk, k2) and ColFrag(Psi
  // tile (kk, j)): each step's maps are loaded two steps ahead, so their
  // latency hides under the two products in between (four steps ahead, with
  // four sets, measured slower: 23-25 against 22 us at G = 8)
  f32x4 phA[NK], psA, phB[NK], psB;
  auto load = [&](int seg, f32x4(&ph)[NK], f32x4 &ps) {
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
  auto seg_of = [&](int step) { return REV ? G - 1 - step : step; };
  // products needed: one per segment, but the forward without S_final needs
  // none for its last segment (whose map need not exist)
  const int nprod = (!REV && !S_final) ? G - 1 : G;
  if (nprod > 0)
    load(seg_of(0), phA, psA);
  if (nprod > 1)
    load(seg_of(1), phB, psB);
  // one step: S_in of the step's segment, then (if needed) the next state;
  // the set it used is refilled with the maps two steps ahead (past the
  // last product: its own maps again, no branch).  False: no more products.
  auto step_fn = [&](int step, f32x4(&ph)[NK], f32x4 &ps) -> bool {
    const int seg = seg_of(step);
    const size_t base = (static_cast<size_t>(seg) * H + h) * D * D;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S_in[base + at(i)] = s[i];
    if (step >= nprod)
      return false;  // uniform over the workgroup
    col[kk][lane] = s;
    lds_barrier();
    f32x4 cph[NK];
#pragma unroll
    for (int k2 = 0; k2 < NK; ++k2)
      cph[k2] = ph[k2];
    f32x4 nw = ps;
    load(seg_of(step + 2 < nprod ? step + 2 : step), ph, ps);
#pragma unroll
    for (int k2 = 0; k2 < NK; ++k2)
      mm<float>(nw, cph[k2], col[k2][lane]);
    lds_barrier();  // every wave has read the column before it is overwritten
    s = nw;
    return true;
  };
  if constexpr (GC > 0) {
#pragma unroll
    for (int step = 0; step < GC; step += 2) {
      if (!step_fn(step, phA, psA))
        break;
      if (step + 1 >= GC || !step_fn(step + 1, phB, psB))
        break;
    }
  } else {
    for (int step = 0; step < G; step += 2) {
      if (!step_fn(step, phA, psA))
        break;
      if (step + 1 >= G || !step_fn(step + 1, phB, psB))
        break;
    }
  }
  if (S_final) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S_final[static_cast<size_t>(bh) * D * D + at(i)] = s[i];
  }
}

template <typename IO, int D, int C, int CW>
hipError_t launch_segmap_cw(const chunk_args &a, float *Phi, float *Psi, hipStream_t st) {
  typedef segmap_cfg<IO, D, C, CW> K;
  const long units_pad = (static_cast<long>(a.num_seqs) * a.H + 7) / 8 * 8;
  hipLaunchKernelGGL((gdn2_segmap_kernel<IO, D, C, CW>), dim3(static_cast<unsigned>(units_pad * K::NPART * K::NSPL)),
                     dim3(64 * (K::NW + K::NL)), 0, st, a, Phi, Psi);
  return hipGetLastError();
}

// Two column tiles per wave once one tile per wave would need more than one
// round of workgroups (two per compute unit); fewer units keep one tile per
// wave and twice the workgroups.
template <typename IO, int D, int C>
hipError_t launch_segmap(const chunk_args &a, float *Phi, float *Psi, hipStream_t st) {
  constexpr int NK = D / 16;
  if constexpr (sizeof(IO) == 2 && NK % 2 == 0) {
    if (static_cast<long>(a.num_seqs) * a.H * NK > 512)
      return launch_segmap_cw<IO, D, C, 2>(a, Phi, Psi, st);
  }
  return launch_segmap_cw<IO, D, C, 1>(a, Phi, Psi, st);
}

template <int D>
hipError_t launch_seg_combine(const float *Phi, const float *Psi, const float *S0, int G, int H, int B,
                              float *S_in, float *S_final, hipStream_t st, bool reverse) {
  const dim3 grid((B * H + 7) / 8 * 8 * (D / 16)), block(64 * (D / 16));
  if (reverse)
    hipLaunchKernelGGL((gdn2_seg_combine_kernel<D, true>), grid, block, 0, st, Phi, Psi, S0, G, H, B, S_in, S_final);
  else if (G == 2 || G == 4 || G == 8 || G == 16) {
    // the segment schedule's counts, unrolled
    if (G == 2)
      hipLaunchKernelGGL((gdn2_seg_combine_kernel<D, false, 2>), grid, block, 0, st, Phi, Psi, S0, G, H, B, S_in,
                         S_final);
    else if (G == 4)
      hipLaunchKernelGGL((gdn2_seg_combine_kernel<D, false, 4>), grid, block, 0, st, Phi, Psi, S0, G, H, B, S_in,
                         S_final);
    else if (G == 8)
      hipLaunchKernelGGL((gdn2_seg_combine_kernel<D, false, 8>), grid, block, 0, st, Phi, Psi, S0, G, H, B, S_in,
                         S_final);
    else
      hipLaunchKernelGGL((gdn2_seg_combine_kernel<D, false, 16>), grid, block, 0, st, Phi, Psi, S0, G, H, B, S_in,
                         S_final);
  } else {
    hipLaunchKernelGGL((gdn2_seg_combine_kernel<D, false>), grid, block, 0, st, Phi, Psi, S0, G, H, B, S_in, S_final);
  }
  return hipGetLastError();
}

// Bounds of G segments of each of B sequences laid end to end: sequence b
// spans [cu[b], cu[b+1]) when cu is given (packed input), else [b T, b T + T).
// Its segments hold ceil(chunks / G) chunks each, the last ones shorter or
// empty: segment g starts at start_b + min(g L_b, len_b).  seg_cu[B G] is the
// end of the last sequence.  With `offsets` it also writes the segments'
// chunk table (as gdn2_chunk_table_kernel would from seg_cu): the segments
// are whole chunks, so segment g of sequence b starts at chunk P_b +
// min(g Lc_b, nc_b), with P_b the chunks of the sequences before b, nc_b
// its own and Lc_b = L_b / C.  One workgroup of 256 threads.
__global__ void __launch_bounds__(256) gdn2_seg_bounds_kernel(const int32_t *__restrict__ cu,
                                                              int32_t *__restrict__ seg_cu, int G, int T, int B,
                                                              int C, int32_t *__restrict__ offsets) {
  auto seq = [&](int b, long &start, long &len, long &nc) {
    start = cu ? static_cast<long>(cu[b]) : static_cast<long>(b) * T;
    len = cu ? static_cast<long>(cu[b + 1]) - cu[b] : static_cast<long>(T);
    nc = (len + C - 1) / C;
  };
  for (int i = static_cast<int>(threadIdx.x); i <= B * G; i += static_cast<int>(blockDim.x)) {
    const int b = i < B * G ? i / G : B - 1, g = i < B * G ? i - b * G : G;
    long start, len, nc;
    seq(b, start, len, nc);
    const long L = (nc + G - 1) / G * C;
    const long x = static_cast<long>(g) * L;
    seg_cu[i] = static_cast<int32_t>(start + (x < len ? x : len));
  }
  if (!offsets)
    return;  // the whole workgroup
  __shared__ int part[256];
  const int tid = static_cast<int>(threadIdx.x);
  const int per = (B + 255) / 256;
  const int beg = tid * per, end = (beg + per < B) ? beg + per : B;
  int sum = 0;
  for (int b = beg; b < end; ++b) {
    long start, len, nc;
    seq(b, start, len, nc);
    sum += static_cast<int>(nc);
  }
  part[tid] = sum;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int i = 0; i < 256; ++i) {
      const int vv = part[i];
      part[i] = acc;
      acc += vv;
    }
    offsets[B * G] = acc;
  }
  __syncthreads();
  int acc = part[tid];
  for (int b = beg; b < end; ++b) {
    long start, len, nc;
    seq(b, start, len, nc);
    const long Lc = (nc + G - 1) / G;
    for (int g = 0; g < G; ++g) {
      const long x = static_cast<long>(g) * Lc;
      offsets[b * G + g] = acc + static_cast<int>(x < nc ? x : nc);
    }
    acc += static_cast<int>(nc);
  }
}

hipError_t launch_seg_bounds(const int32_t *cu, int32_t *seg_cu, int G, int T, int B, int C, hipStream_t st,
                             int32_t *offsets) {
  if (G < 1 || B < 1 || C < 1)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(gdn2_seg_bounds_kernel, dim3(1), dim3(256), 0, st, cu, seg_cu, G, T, B, C, offsets);
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
