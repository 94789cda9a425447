// gdn2_chunk.hip -- two-pass chunkwise GDN-2 forward for gfx950.
//
// Pass 1 (gdn2_chunk_prep_kernel) runs the per-chunk phases of gdn2_wy.hpp for
// every (chunk, head) in parallel and writes the chunk's -W, Q', Kbar^T,
// gamma_C, P's lower-triangular tiles and Ut to the workspace in fragment
// order.  Pass 2 (gdn2_chunk_scan_kernel) walks the chunks of each sequence
// in order with the state in matrix-core accumulators and forms
// O_intra = P Ut on the way.  This path keeps the whole GPU busy
// when there are few (sequence, head) units (long sequences, small batch);
// gdn2_fused.hip does both passes in one workgroup per head and avoids the
// workspace round trip when there are enough units.  gdn2_chunk_table_kernel
// builds the per-sequence chunk offsets of packed input.
#include "gdn2_wy.hpp"

#include <type_traits>

namespace gdn2 {

template <typename IO, int D, int C> size_t chunk_block_bytes() { return blk_layout<IO, D, C>::BYTES; }

// Pass 1.  grid: num_slots * H, block: 64 * C/16 threads (see gdn2_wy.hpp for
// the work split between waves).
template <typename IO, int D, int C, int GM>
__global__ void __launch_bounds__(64 * (C / 16)) __attribute__((amdgpu_waves_per_eu(2)))
gdn2_chunk_prep_kernel(chunk_args a) {
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

  constexpr bool LP = GM == GM_LAYER;
  wy_rows<IO, D, LP> r;
  raw4<IO> rv[NB][CTW], rw[NB][CTW];
  wy_load_chunk<IO, D, C, CTW, GM>(a, t0, len, h, I, ct0, owner, m, g, r, rv, rw);
  f32x4 gl[NK];
  bool pw;
  wy_decay<IO, D, C, LP>(sm, r, gl, pw, a, t0, len, h, I, tid, reinterpret_cast<float *>(blk + L::GAM));
  const F eye = identity_colfrag<IO>(lane);
  wy_ops<IO, D> op;
  wy_operands<IO, D, C, LP>(sm, r, gl, pw, a, t0, len, h, I, lane, eye, blk + L::KB, op);
  F ucol[NB][CTW];
  wy_values<IO, NB, CTW, LP>(rv, rw, eye, ucol);
  __syncthreads();
  F af[NB];
  wy_products<IO, D, C>(sm, op, I, lane, af);
  wy_inverse<IO, D, C>(sm, af, I, lane, eye);
  // P's tiles of this wave's rows (complete in LDS since wy_inverse's
  // barriers), for the scan to form O_intra = P Ut
#pragma unroll
  for (int J = 0; J < NB; ++J)
    if (J <= I)
      F::ld(sm.pr[tri_index(I, J)], lane).st(blk + L::P + static_cast<size_t>(tri_index(I, J)) * L::TB, lane);
  if (owner) {
    wy_tp<IO, C> tp;
    wy_load_tp<IO, D, C>(sm, lane, tp);
    F ut[CTW][NB];
#pragma unroll
    for (int j = 0; j < CTW; ++j) {
      const int ct = ct0 + j;
      wy_wq<IO, D, C>(sm, tp, ct, lane, eye, blk + L::WN, blk + L::QP);
      F uc_j[NB];
#pragma unroll
      for (int J = 0; J < NB; ++J)
        uc_j[J] = ucol[J][j];
      f32x4 u4[NB], o4[NB];
      wy_uo<IO, C, true, false>(tp, uc_j, u4, o4);
#pragma unroll
      for (int I2 = 0; I2 < NB; ++I2)
        ut[j][I2] = F::from(u4[I2]);
    }
#pragma unroll
    for (int I2 = 0; I2 < NB; ++I2) {
      if constexpr (CTW % 2 == 0 && NK % 2 == 0) {
#pragma unroll
        for (int j = 0; j < CTW; j += 2)  // ct0 is even: one 16-byte store per tile pair
          frag2<IO>::make(ut[j][I2], ut[j + 1][I2]).st(blk + L::UT + tile_off<IO, NK>(I2, ct0 + j, 0), lane);
      } else {
#pragma unroll
        for (int j = 0; j < CTW; ++j)
          ut[j][I2].st_at(blk + L::UT + tile_off<IO, NK>(I2, ct0 + j, lane));
      }
    }
  }
}

// Work split of the state scan for one (sequence, head): the dv tiles go to
// NGRP = NK / NT workgroups of NT tiles each (NT is chosen at launch from the
// number of units), each with NCW compute waves of CPW 16-column state slices
// and NLW loader waves.  Each LDS buffer holds the SHARED part of one chunk's
// block (P's tiles included) and, when a tile row of the workgroup's columns
// is a whole number of KB (UO_LDS), the workgroup's Ut tiles (rows tt, TF
// tiles each: its NT tiles rounded out to whole stored pairs).  R1: the
// block of rule R1, whose shared part ends at SHARED0 (no P) and whose -Ut'
// and O'' rows are both staged; one column tile per compute wave.  ST
// (states mode): the output's operands Q' and P are not copied, only -W,
// Kbar^T, gamma_C and the Ut rows (the LDS keeps the block's offsets).
template <typename IO, int D, int C, int NT, bool R1 = false, bool ST = false> struct scan_cfg {
  typedef blk_layout<IO, D, C> L;
  static constexpr int NB = C / 16, NK = D / 16;
  static_assert(NT >= 1 && NT <= NK && NK % NT == 0, "tiles per workgroup");
  // two column tiles per compute wave at NT = 2 (one compute wave per
  // workgroup); at NT = 4 two such waves would spill, four waves of one tile
  // do not, and rule R1's N tiles need the room
  static constexpr int CPW = (sizeof(IO) == 2 && NT == 2 && !R1) ? 2 : 1;
  static constexpr int NCW = NT / CPW;
  static constexpr int NGRP = NK / NT;
  static constexpr int NTW = NT;                     // dv tiles per workgroup
  // tiles staged per row: the workgroup's tiles rounded out to whole pairs
  // (dv tiles are stored paired when NK is even)
  static constexpr int TF = (NK % 2 == 0) ? (NT + 1) / 2 * 2 : NT;
  static constexpr size_t RB = TF * L::TB;           // one staged tile row of Ut
  static constexpr bool UO_LDS = RB % 1024 == 0;
  static constexpr int RPP = static_cast<int>(RB / 1024);
  static constexpr size_t SHR = R1 ? L::SHARED0 : L::SHARED;  // shared part of the block
  static constexpr int NRW = R1 ? 2 : 1;                        // staged row regions: Ut (and O'')
  static_assert(!R1 || UO_LDS, "rule R1 stages its -Ut' and O'' rows");
  static constexpr size_t BUF = SHR + (UO_LDS ? NRW * NB * RB : 0);
  static constexpr int NPS = static_cast<int>(SHR / 1024);
  // states mode: the Q' pieces [QP, KB) are skipped when they are whole KB,
  // and the P pieces [SHARED0, SHARED) always (SHARED0 is a whole KB)
  static constexpr bool SKIPQ = ST && L::QP % 1024 == 0 && L::KB % 1024 == 0;
  static constexpr int NQS = SKIPQ ? static_cast<int>((L::KB - L::QP) / 1024) : 0;
  static constexpr int NPS_LD = ST ? static_cast<int>(L::SHARED0 / 1024) - NQS : NPS;  // shared pieces copied
  static constexpr int NPIECE = NPS_LD + static_cast<int>((BUF - SHR) / 1024);         // 1 KB per wave load
  static constexpr int NLW = NPIECE < 4 ? NPIECE : (NPIECE + 12) / 13 > 4 ? (NPIECE + 12) / 13 : 4;
  static constexpr int PPW = (NPIECE + NLW - 1) / NLW;         // pieces per loader wave
  static constexpr int RSETS = PPW <= 16 ? 2 : 1;              // loader register buffers
  static constexpr int NBUF = (2 * BUF <= 160 * 1024) ? 2 : 1;
};

// Pass 2: sequential state scan + output.  For chunk c of a (sequence, head):
//   Z = Ut - W S,  O = P Ut + Q' S  (written to o),  S <- Diag(gamma_C) S + Kbar^T Z.
// Every 16-column slice of S evolves on its own given the chunk's -W, Q',
// Kbar^T, gamma_C and P (the SHARED part of the block), so the dv columns are
// split over NGRP workgroups x NCW compute waves, each keeping its CPW slices
// of S (dk x 16, float32) in matrix-core accumulators for the whole sequence.
// NLW loader waves move each chunk's operands (62 KB for a workgroup of four
// column tiles, bf16, d = 128, C = 64: the 54 KB shared part and 8 KB of Ut)
// HBM -> registers -> LDS two chunks ahead of the compute waves (one
// LDS buffer ahead, one register set ahead), so that the wide loads are
// spread over several waves and never stall the waves doing the products; a
// compute wave issues no global load inside the loop.  O is accumulated
// transposed (O^T = S^T Q'^T, the same registers with the operands swapped),
// which leaves four consecutive columns of one row in each lane: one 8-byte
// store per lane and tile.  One LDS-only barrier per chunk (two with a single
// LDS buffer); global stores are never waited for inside the loop, and the
// body of a full chunk has no branch.
// Grid: units_pad * NGRP workgroups, units_pad = N*H rounded up to 8;
// consecutive ids go to the 8 XCDs round-robin and all workgroups of one head
// share an XCD (and its L2).
// With ST (states mode, used by the backward) the kernel writes, instead of
// o, the state entering every chunk to a.states (chunk slot order, one
// state_tiles block per chunk-head: fragment tiles of the I/O type).
// With WS (keep states) the forward scan also writes the state entering
// every chunk to a.states, as the states mode does, next to o: a training
// step's forward hands them to the backward.  The state entering chunk
// c + 1 is stored right after chunk c's update, where the output's
// registers are dead (before the chunk it would raise the register peak).
// With R1 it scans the blocks of rule R1 (r1_layout): O starts from the
// stored O'' instead of P Ut, and the update adds the chunk's N tiles, which
// each compute wave reads from the block at the start of the chunk:
//   Z = -Ut' - W' S,  O = Q'' S + O'',  S <- Diag(gamma_C) S + Ebar^T Z + N.
template <typename IO, int D, int C, int NT, bool ST = false, bool R1 = false, bool WS = false>
__global__ void __launch_bounds__(64 * (scan_cfg<IO, D, C, NT, R1, ST>::NCW + scan_cfg<IO, D, C, NT, R1, ST>::NLW))
    gdn2_chunk_scan_kernel(chunk_args a) {
  typedef scan_cfg<IO, D, C, NT, R1, ST> K;
  typedef r1_layout<IO, D, C> R;
  static_assert(!(ST && R1), "rule R1 has no states mode");
  static_assert(!R1 || (sizeof(IO) == 2 && (D / 16) % 2 == 0 && (C / 16) % 2 == 0),
                "rule R1 takes the bfloat16 paired-tile form");
  constexpr int NB = C / 16, NK = D / 16;
  constexpr int NCW = K::NCW, CPW = K::CPW, NGRP = K::NGRP, NLW = K::NLW, PPW = K::PPW, NTW = K::NTW,
                TF = K::TF;
  constexpr int NPIECE = K::NPIECE, NPS_LD = K::NPS_LD, RPP = K::RPP, NBUF = K::NBUF;
  constexpr size_t RB = K::RB;
  typedef frag<IO> F;
  typedef frag2<IO> F2;
  typedef blk_layout<IO, D, C> L;
  typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
  __shared__ __attribute__((aligned(16))) unsigned char sbuf[NBUF][K::BUF];

  const int x = blockIdx.x;
  const int xcd = x & 7, s8 = x >> 3;
  const int unit = (s8 / NGRP) * 8 + xcd;
  const int grp = s8 % NGRP;
  if (unit >= a.num_seqs * a.H)
    return;  // whole workgroup
  const int n = unit / a.H, h = unit - n * a.H;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int vtg = grp * NTW;                          // first dv tile of the workgroup
  const int vtf = (NK % 2 == 0) ? (vtg & ~1) : vtg;   // first staged dv tile
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

  if (wave >= NCW) {
    // ---- loader wave: pieces lw, lw + NLW, ... of an LDS buffer
    if (nchunks == 0)
      return;  // the compute waves take no barrier either
    const int lw = wave - NCW;
    // byte offset in the block of LDS piece p (the shared part, then Ut
    // rows, then for R1 the O'' rows; the row pieces exist only when UO_LDS,
    // i.e. RPP >= 1), and its offset in an LDS buffer: a shared piece keeps
    // its block offset (states mode skips the Q' pieces), the row pieces
    // follow the shared part
    auto piece_src = [&](int p) -> size_t {
      constexpr int RP = RPP > 0 ? RPP : 1;
      if (p < NPS_LD)
        return static_cast<size_t>(p >= static_cast<int>(L::QP / 1024) ? p + K::NQS : p) * 1024;
      int q = p - NPS_LD;
      size_t base = R1 ? R::UT : L::UT;
      if (R1 && q >= NB * RP) {
        q -= NB * RP;
        base = R::OI;
      }
      return base + tile_off<IO, NK>(q / RP, vtf, 0) + static_cast<size_t>(q % RP) * 1024;
    };
    auto piece_dst = [&](int p) -> int {
      if (p < NPS_LD)
        return static_cast<int>(piece_src(p));
      return static_cast<int>(K::SHR) + (p - NPS_LD) * 1024;
    };
    int src_off[PPW], dst_off[PPW];
#pragma unroll
    for (int p = 0; p < PPW; ++p) {
      const int piece = lw + p * NLW;
      src_off[p] = piece < NPIECE ? static_cast<int>(piece_src(piece)) : 0;
      dst_off[p] = piece < NPIECE ? piece_dst(piece) : 0;
    }
    u32x4 ra[PPW], rb[PPW];
    // Always issues PPW loads (past the last chunk: the first bytes of the
    // last block again) so the number of loads in flight is fixed.
    auto gload = [&](int c, u32x4(&r)[PPW]) {
      const bool valid = c < nchunks;
      const unsigned char *src = blk_of(valid ? c : nchunks - 1);
#pragma unroll
      for (int p = 0; p < PPW; ++p)
        r[p] = *reinterpret_cast<const u32x4 *>(src + (valid ? src_off[p] : 0) + lane * 16);
    };
    auto lstore = [&](int buf, const u32x4(&r)[PPW]) {
#pragma unroll
      for (int p = 0; p < PPW; ++p) {
        const int piece = lw + p * NLW;
        if (piece < NPIECE)
          *reinterpret_cast<u32x4 *>(&sbuf[buf][dst_off[p] + lane * 16]) = r[p];
      }
    };
    gload(0, ra);
    lstore(0, ra);
    if constexpr (K::RSETS == 2) {
      gload(1, rb);
      lds_barrier();  // chunk 0 is in buffer 0
      for (int c = 0; c < nchunks; c += 2) {
        gload(c + 2, ra);  // ra held chunk c (already in LDS)
        if constexpr (NBUF == 1)
          lds_barrier();  // compute waves are done with the only buffer
        if (c + 1 < nchunks)
          lstore((c + 1) % NBUF, rb);
        lds_barrier();  // chunk c + 1 is in LDS, chunk c's buffer is free
        if (c + 1 >= nchunks)
          break;
        gload(c + 3, rb);
        if constexpr (NBUF == 1)
          lds_barrier();
        if (c + 2 < nchunks)
          lstore((c + 2) % NBUF, ra);
        lds_barrier();
      }
    } else {
      lds_barrier();
      for (int c = 0; c < nchunks; ++c) {
        gload(c + 1, ra);
        if constexpr (NBUF == 1)
          lds_barrier();
        if (c + 1 < nchunks)
          lstore((c + 1) % NBUF, ra);
        lds_barrier();
      }
    }
    return;
  }

  // ---- compute wave: dv tiles vt0 .. vt0 + CPW - 1
  const int m = lane & 15, g = lane >> 4;
  const F eye = identity_colfrag<IO>(lane);
  const int vt0 = vtg + wave * CPW;
  f32x4 S[NK][CPW];
  if (a.S0) {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[kk][j][i] = a.S0[(static_cast<size_t>(unit) * D + 16 * kk + 4 * g + i) * D + 16 * (vt0 + j) + m];
  } else {
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int j = 0; j < CPW; ++j)
        S[kk][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Ut tiles of chunk c from global memory (when they are not staged in
  // LDS; past the last chunk: the last again)
  auto tload = [&](int c, F(&u)[NB][CPW]) {
    const unsigned char *blk = blk_of(c < nchunks ? c : nchunks - 1);
#pragma unroll
    for (int tt = 0; tt < NB; ++tt)
#pragma unroll
      for (int j = 0; j < CPW; ++j)
        u[tt][j] = F::ld_at(blk + L::UT + tile_off<IO, NK>(tt, vt0 + j, lane));
  };
  // Ut tile (row tile J, column slice j): from an LDS buffer (UO_LDS), read
  // at its use, or from the registers tload filled
  auto u_tile = [&](const unsigned char *sb, const F(&ucur)[NB][CPW], int J, int j) -> F {
    if constexpr (K::UO_LDS)
      return F::ld_at(sb + K::SHR + J * RB + tile_off<IO, TF>(0, vt0 + j - vtf, lane));
    else
      return ucur[J][j];
  };
  // O_intra^T of row tile tt, column slice j: sum over J <= tt of
  // Ut(J)^T P(tt, J)^T (operands swapped as in the prep: RowFrag(O_intra)),
  // in the product shape of the rest of the output chain -- PAIR: 16x16x32
  // over pairs of J (a missing partner is a zero tile), else single tiles.
  auto o_intra = [&](const unsigned char *sb, const F(&ucur)[NB][CPW], int tt, int j, auto pair) -> f32x4 {
    constexpr bool PAIR = decltype(pair)::value;
    auto ptile = [&](int J) { return F::ld(sb + L::P + static_cast<size_t>(tri_index(tt, J)) * L::TB, lane); };
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    if constexpr (PAIR) {
#pragma unroll
      for (int J = 0; J < NB; J += 2) {
        if (J <= tt) {
          const bool two = J + 1 <= tt && J + 1 < NB;
          mma32(o, F2::make(u_tile(sb, ucur, J, j), two ? u_tile(sb, ucur, J + 1, j) : F::zero()),
                F2::make(ptile(J), two ? ptile(J + 1) : F::zero()));
        }
      }
    } else {
#pragma unroll
      for (int J = 0; J < NB; ++J)
        if (J <= tt)
          mm_io(o, u_tile(sb, ucur, J, j), ptile(J));
    }
    return o;
  };

  // One chunk: products, o stores (rows < len unless FULL) and state update.
  auto chunk_step = [&](const unsigned char *sb, const F(&ucur)[NB][CPW], long t0, int len, int c, auto full) {
    constexpr bool FULL = decltype(full)::value;
    if constexpr (ST) {
      typedef state_tiles<IO, D> ST_;
      unsigned char *sp =
          reinterpret_cast<unsigned char *>(a.states) + (static_cast<size_t>(c_begin + c) * a.H + h) * ST_::BYTES;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
          const F sc = F::from(S[kk][j]);  // ColFrag(S tile (kk, vt0 + j))
          sc.st(sp + ST_::COL + ST_::off(kk, vt0 + j), lane);
          if constexpr (ST_::HAS_ROW)
            F::from(transpose_io(sc, eye, lane)).st(sp + ST_::ROW + ST_::off(kk, vt0 + j), lane);
        }
    }
    // o goes through a global-address-space pointer so that the compiler
    // knows these stores never alias the LDS operands it wants to hoist
    typedef __attribute__((address_space(1))) typename io<IO>::elem gelem;
    gelem *gout = (gelem *)(a.o);
    F sf[NK][CPW];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int j = 0; j < CPW; ++j)
        sf[kk][j] = F::from(S[kk][j]);
    F zf[NB][CPW];
    if constexpr (NK % 2 == 0 && NB % 2 == 0 && CPW == 1) {
      // (one column tile per wave: with two, these registers would spill)
      // Every product chain is short (NK / 2 steps for Z and O, NB / 2 for
      // the update) and a dependent step costs several times an issue slot,
      // so the loops run the k-pairs outermost: each step advances the
      // chains of all row tiles (Z and O) or of a group of GK row tiles (the
      // update), whose products are independent and fill each other's wait.
      f32x4 z[NB][CPW], ot[NB][CPW];
      // R1: this wave's N tiles of the chunk, in flight during the products
      F ntile[R1 ? NK : 1][CPW];
      if constexpr (R1) {
        const unsigned char *blk = blk_of(c);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk)
#pragma unroll
          for (int j = 0; j < CPW; ++j)
            ntile[kk][j] = F::ld_at(blk + R::NC + tile_off<IO, NK>(kk, vt0 + j, lane));
      }
#pragma unroll
      for (int tt = 0; tt < NB; ++tt) {
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
          const F ut = u_tile(sb, ucur, tt, j);
          if constexpr (sizeof(IO) == 2) {
            // start from Ut with an identity product instead of unpacking
            // bf16 on the vector ALU (which the products wait for); same
            // product shape as the rest of the chain (see mma32)
            z[tt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            mma32(z[tt][j], F2::make(eye, F::zero()), F2::make(ut, ut));
            if constexpr (R1) {
              // O''^T of row tile tt from the staged rows after the Ut rows
              const F oi = F::ld_at(sb + K::SHR + (NB + tt) * RB + tile_off<IO, TF>(0, vt0 + j - vtf, lane));
              ot[tt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
              mma32(ot[tt][j], F2::make(eye, F::zero()), F2::make(oi, oi));
            } else {
              ot[tt][j] = o_intra(sb, ucur, tt, j, std::true_type{});
            }
          } else {
            z[tt][j] = ut.to_f32();
            ot[tt][j] = o_intra(sb, ucur, tt, j, std::false_type{});
          }
        }
      }
      // -W and Q' pairs of k-pair k2 for every row tile, two register
      // buffers: pair k2 + 1 is read while k2 is multiplied
      F2 w2[2][NB], q2[2][NB];
      auto wq_pair = [&](int k2, int b) {
#pragma unroll
        for (int tt = 0; tt < NB; ++tt) {
          w2[b][tt] = F2::ld(sb + L::WN + tile_off<IO, NK>(tt, 2 * k2, 0), lane);
          q2[b][tt] = F2::ld(sb + L::QP + tile_off<IO, NK>(tt, 2 * k2, 0), lane);
        }
      };
      wq_pair(0, 0);
#pragma unroll
      for (int k2 = 0; k2 < NK / 2; ++k2) {
        if (k2 + 1 < NK / 2)
          wq_pair(k2 + 1, (k2 + 1) % 2);
#pragma unroll
        for (int tt = 0; tt < NB; ++tt)
#pragma unroll
          for (int j = 0; j < CPW; ++j) {
            const F2 s2 = F2::make(sf[2 * k2][j], sf[2 * k2 + 1][j]);
            mma32(z[tt][j], w2[k2 % 2][tt], s2);
            mma32(ot[tt][j], s2, q2[k2 % 2][tt]);
          }
      }
#pragma unroll
      for (int tt = 0; tt < NB; ++tt) {
        const int t = 16 * tt + m;  // this lane's row of the O tile
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
          zf[tt][j] = F::from(z[tt][j]);
          if (!ST && (FULL || t < len))
            store4_global(gout + (static_cast<size_t>(t0 + t) * a.H + h) * D + 16 * (vt0 + j) + 4 * g, ot[tt][j]);
        }
      }
      // S <- Diag(gamma_C) S + Kbar^T Z, GK row tiles at a time
      constexpr int GK = NK;
#pragma unroll
      for (int k0 = 0; k0 < NK; k0 += GK) {
        f32x4 gamv[GK];
        F2 kbp[GK][NB / 2];
#pragma unroll
        for (int u = 0; u < GK; ++u) {
          gamv[u] = *reinterpret_cast<const f32x4 *>(sb + L::GAM + (16 * (k0 + u) + 4 * g) * sizeof(float));
#pragma unroll
          for (int t2 = 0; t2 < NB / 2; ++t2)
            kbp[u][t2] = F2::ld(sb + L::KB + tile_off<IO, NB>(k0 + u, 2 * t2, 0), lane);
        }
#pragma unroll
        for (int u = 0; u < GK; ++u)
#pragma unroll
          for (int j = 0; j < CPW; ++j) {
            S[k0 + u][j] *= gamv[u];
            if constexpr (R1)  // + N, by an identity product (exact in float32)
              mma32(S[k0 + u][j], F2::make(eye, F::zero()), F2::make(ntile[k0 + u][j], ntile[k0 + u][j]));
          }
#pragma unroll
        for (int t2 = 0; t2 < NB / 2; ++t2)
#pragma unroll
          for (int u = 0; u < GK; ++u)
#pragma unroll
            for (int j = 0; j < CPW; ++j)
              mma32(S[k0 + u][j], kbp[u][t2], F2::make(zf[2 * t2][j], zf[2 * t2 + 1][j]));
      }
    } else {
      // LDS operands of the state update (gamma_C and the Kbar^T pairs of row
      // tile kk), in two register buffers: row tile kk + 1 is read while kk is
      // multiplied, and row tile 0 during the products above (read at their
      // use, each row tile waited a full LDS round trip)
      constexpr int NKB = NB % 2 == 0 ? NB / 2 : 1;
      f32x4 gamv[2];
      F2 kbp[2][NKB];
      auto su_load = [&](int kk, int b) {
        gamv[b] = *reinterpret_cast<const f32x4 *>(sb + L::GAM + (16 * kk + 4 * g) * sizeof(float));
        if constexpr (NB % 2 == 0) {
  #pragma unroll
          for (int t2 = 0; t2 < NKB; ++t2)
            kbp[b][t2] = F2::ld(sb + L::KB + tile_off<IO, NB>(kk, 2 * t2, 0), lane);
        }
      };
      // -W and Q' pairs of row tile tt, two register buffers: tile tt + 1 is
      // read while tile tt is multiplied (one column tile per wave; with two,
      // the extra registers would spill and the pairs are read at their use)
      constexpr bool WQ_PF = CPW == 1;
      constexpr int NKP = NK % 2 == 0 ? NK / 2 : 1;
      F2 wq_w[WQ_PF ? 2 : 1][NKP], wq_q[WQ_PF ? 2 : 1][NKP];
      auto wq_load = [&](int tt, F2(&w)[NKP], F2(&q)[NKP]) {
        if constexpr (NK % 2 == 0 && WQ_PF) {
  #pragma unroll
          for (int k2 = 0; k2 < NKP; ++k2) {
            w[k2] = F2::ld(sb + L::WN + tile_off<IO, NK>(tt, 2 * k2, 0), lane);
            q[k2] = F2::ld(sb + L::QP + tile_off<IO, NK>(tt, 2 * k2, 0), lane);
          }
        }
      };
      wq_load(0, wq_w[0], wq_q[0]);
  #pragma unroll
      for (int tt = 0; tt < NB; ++tt) {
        if (tt + 1 < NB)
          wq_load(tt + 1, wq_w[WQ_PF ? (tt + 1) % 2 : 0], wq_q[WQ_PF ? (tt + 1) % 2 : 0]);
        else
          su_load(0, 0);
        f32x4 z[CPW], ot[CPW];
  #pragma unroll
        for (int j = 0; j < CPW; ++j) {
          const F ut = u_tile(sb, ucur, tt, j);
          if constexpr (sizeof(IO) == 2) {
            // start from Ut with an identity product instead of unpacking
            // bf16 on the vector ALU (which the products wait for); same
            // product shape as the rest of the chain (see mma32)
            z[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (NK % 2 == 0) {
              mma32(z[j], F2::make(eye, F::zero()), F2::make(ut, ut));
              ot[j] = o_intra(sb, ucur, tt, j, std::true_type{});
            } else {
              mma16(z[j], eye, ut);
              ot[j] = o_intra(sb, ucur, tt, j, std::false_type{});
            }
          } else {
            z[j] = ut.to_f32();
            ot[j] = o_intra(sb, ucur, tt, j, std::false_type{});
          }
        }
        if constexpr (NK % 2 == 0) {
  #pragma unroll
          for (int k2 = 0; k2 < NK / 2; ++k2) {
            const F2 w2 = WQ_PF ? wq_w[tt % 2][k2] : F2::ld(sb + L::WN + tile_off<IO, NK>(tt, 2 * k2, 0), lane);
            const F2 q2 = WQ_PF ? wq_q[tt % 2][k2] : F2::ld(sb + L::QP + tile_off<IO, NK>(tt, 2 * k2, 0), lane);
  #pragma unroll
            for (int j = 0; j < CPW; ++j) {
              const F2 s2 = F2::make(sf[2 * k2][j], sf[2 * k2 + 1][j]);
              mma32(z[j], w2, s2);
              mma32(ot[j], s2, q2);
            }
          }
        } else {
  #pragma unroll
          for (int kk = 0; kk < NK; ++kk) {
            const F w1 = F::ld(sb + L::WN + tile_off<IO, NK>(tt, kk, 0), lane);
            const F q1 = F::ld(sb + L::QP + tile_off<IO, NK>(tt, kk, 0), lane);
  #pragma unroll
            for (int j = 0; j < CPW; ++j) {
              mma16(z[j], w1, sf[kk][j]);
              mma16(ot[j], sf[kk][j], q1);
            }
          }
        }
        const int t = 16 * tt + m;  // this lane's row of the O tile
  #pragma unroll
        for (int j = 0; j < CPW; ++j) {
          zf[tt][j] = F::from(z[j]);
          if (!ST && (FULL || t < len))
            store4_global(gout + (static_cast<size_t>(t0 + t) * a.H + h) * D + 16 * (vt0 + j) + 4 * g, ot[j]);
        }
      }
  #pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        if (kk + 1 < NK)
          su_load(kk + 1, (kk + 1) % 2);
  #pragma unroll
        for (int j = 0; j < CPW; ++j)
          S[kk][j] *= gamv[kk % 2];
        if constexpr (NB % 2 == 0) {
  #pragma unroll
          for (int t2 = 0; t2 < NB / 2; ++t2) {
  #pragma unroll
            for (int j = 0; j < CPW; ++j)
              mma32(S[kk][j], kbp[kk % 2][t2], F2::make(zf[2 * t2][j], zf[2 * t2 + 1][j]));
          }
        } else {
  #pragma unroll
          for (int tt = 0; tt < NB; ++tt) {
            const F kb1 = F::ld(sb + L::KB + tile_off<IO, NB>(kk, tt, 0), lane);
  #pragma unroll
            for (int j = 0; j < CPW; ++j)
              mma16(S[kk][j], kb1, zf[tt][j]);
          }
        }

    }
    }
  };

  // WS: the state entering chunk c (slot c_begin + c) as state_tiles
  auto keep_state = [&](int c) {
    if constexpr (WS) {
      typedef state_tiles<IO, D> ST_;
      unsigned char *sp =
          reinterpret_cast<unsigned char *>(a.states) + (static_cast<size_t>(c_begin + c) * a.H + h) * ST_::BYTES;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk)
#pragma unroll
        for (int j = 0; j < CPW; ++j) {
          const F sc = F::from(S[kk][j]);  // ColFrag(S tile (kk, vt0 + j))
          sc.st(sp + ST_::COL + ST_::off(kk, vt0 + j), lane);
          if constexpr (ST_::HAS_ROW)
            F::from(transpose_io(sc, eye, lane)).st(sp + ST_::ROW + ST_::off(kk, vt0 + j), lane);
        }
    }
  };
  if (nchunks > 0) {
    F ucur[NB][CPW];
    if constexpr (!K::UO_LDS)
      tload(0, ucur);
    keep_state(0);
    lds_barrier();  // chunk 0 is in buffer 0
    for (int c = 0; c < nchunks; ++c) {
      const unsigned char *sb = sbuf[c % NBUF];
      const long t0 = tstart + static_cast<long>(c) * C;
      const int len = (tend - t0) < C ? static_cast<int>(tend - t0) : C;
      F unxt[NB][CPW];
      if constexpr (!K::UO_LDS)
        tload(c + 1, unxt);
      if (len == C)
        chunk_step(sb, ucur, t0, len, c, std::true_type{});
      else
        chunk_step(sb, ucur, t0, len, c, std::false_type{});
      if (c + 1 < nchunks)
        keep_state(c + 1);
      if constexpr (NBUF == 1)
        lds_barrier();  // done with the only buffer
      lds_barrier();    // chunk c + 1 is in LDS
      if constexpr (!K::UO_LDS) {
#pragma unroll
        for (int tt = 0; tt < NB; ++tt)
#pragma unroll
          for (int j = 0; j < CPW; ++j)
            ucur[tt][j] = unxt[tt][j];
      }
    }
  }
  // S_final of the sequence (segment schedule: of the original sequence,
  // from its last segment only)
  if (a.S_final && (a.seg_G == 0 || n % a.seg_G == a.seg_G - 1)) {
    const size_t fu = a.seg_G > 0 ? static_cast<size_t>(n / a.seg_G) * a.H + h : static_cast<size_t>(unit);
#pragma unroll
    for (int kk = 0; kk < NK; ++kk)
#pragma unroll
      for (int j = 0; j < CPW; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a.S_final[(fu * D + 16 * kk + 4 * g + i) * D + 16 * (vt0 + j) + m] = S[kk][j][i];
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
  if (a.num_slots > 0) {
    const dim3 grid(a.num_slots * a.H), block(64 * (C / 16));
    const uint32_t kda = GATE_SCALAR_B | GATE_SCALAR_W;
    if (a.gates & GATE_LAYER_PREP)
      hipLaunchKernelGGL((gdn2_chunk_prep_kernel<IO, D, C, GM_LAYER>), grid, block, 0, st, a);
    else if (a.gates == kda)
      hipLaunchKernelGGL((gdn2_chunk_prep_kernel<IO, D, C, GM_KDA>), grid, block, 0, st, a);
    else if (a.gates == (kda | GATE_SCALAR_ALPHA))
      hipLaunchKernelGGL((gdn2_chunk_prep_kernel<IO, D, C, GM_GDN>), grid, block, 0, st, a);
    else if (a.gates)
      hipLaunchKernelGGL((gdn2_chunk_prep_kernel<IO, D, C, GM_GATES>), grid, block, 0, st, a);
    else
      hipLaunchKernelGGL((gdn2_chunk_prep_kernel<IO, D, C, GM_PLAIN>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <typename IO, int D, int C, int NT, bool ST, bool R1 = false, bool WS = false>
hipError_t launch_scan_nt(const chunk_args &a, hipStream_t st) {
  typedef scan_cfg<IO, D, C, NT, R1, ST> K;
  const int units = a.num_seqs * a.H;
  const int units_pad = (units + 7) / 8 * 8;
  hipLaunchKernelGGL((gdn2_chunk_scan_kernel<IO, D, C, NT, ST, R1, WS>), dim3(units_pad * K::NGRP),
                     dim3(64 * (K::NCW + K::NLW)), 0, st, a);
  return hipGetLastError();
}

// Every workgroup takes a whole compute unit (its LDS buffers), so the
// columns of a head are split as finely as the 256 compute units allow: few
// (sequence, head) units get more, narrower workgroups, which shortens the
// sequential per-chunk path; many units get 4 tiles per workgroup.
// float32 inputs with d = 128, C = 64 keep one tile per workgroup: their
// wider fragments would not fit in the registers of the larger workgroups.
template <typename IO, int D, int C, bool ST, bool R1 = false, bool WS = false>
hipError_t launch_scan_any(const chunk_args &a, hipStream_t st) {
  constexpr int NK = D / 16;
  const long units = static_cast<long>(a.num_seqs) * a.H;
  if constexpr (sizeof(IO) == 4 && D * C >= 128 * 64) {
    return launch_scan_nt<IO, D, C, 1, ST, R1, WS>(a, st);
  } else {
    if (units * NK <= 256)
      return launch_scan_nt<IO, D, C, 1, ST, R1, WS>(a, st);
    if constexpr (NK >= 2) {
      if (NK < 4 || units * (NK / 2) <= 256)
        return launch_scan_nt<IO, D, C, 2, ST, R1, WS>(a, st);
    }
    if constexpr (NK >= 4)
      return launch_scan_nt<IO, D, C, 4, ST, R1, WS>(a, st);
    return launch_scan_nt<IO, D, C, 1, ST, R1, WS>(a, st);
  }
}

template <typename IO, int D, int C> hipError_t launch_chunk_scan(const chunk_args &a, hipStream_t st) {
  return launch_scan_any<IO, D, C, false>(a, st);
}

template <typename IO, int D, int C> hipError_t launch_chunk_states(const chunk_args &a, hipStream_t st) {
  return launch_scan_any<IO, D, C, true>(a, st);
}

template <typename IO, int D, int C> hipError_t launch_chunk_scan_keep(const chunk_args &a, hipStream_t st) {
  return launch_scan_any<IO, D, C, false, false, true>(a, st);
}

template <typename IO, int D, int C> hipError_t launch_chunk_scan_r1(const chunk_args &a, hipStream_t st) {
  if constexpr (scan_r1_supported<IO, D, C>())
    return launch_scan_any<IO, D, C, false, true>(a, st);
  else
    return hipErrorNotSupported;
}

hipError_t launch_chunk_table(const int32_t *cu, int N, int C, int32_t *offsets, hipStream_t st) {
  hipLaunchKernelGGL(gdn2_chunk_table_kernel, dim3(1), dim3(256), 0, st, cu, N, C, offsets);
  return hipGetLastError();
}

#define GDN2_INST_CHUNK(IO, D, C)                                                           \
  template size_t chunk_block_bytes<IO, D, C>();                                            \
  template hipError_t launch_chunk_prep<IO, D, C>(const chunk_args &, hipStream_t);         \
  template hipError_t launch_chunk_scan<IO, D, C>(const chunk_args &, hipStream_t);        \
  template hipError_t launch_chunk_states<IO, D, C>(const chunk_args &, hipStream_t);       \
  template hipError_t launch_chunk_scan_keep<IO, D, C>(const chunk_args &, hipStream_t);    \
  template hipError_t launch_chunk_scan_r1<IO, D, C>(const chunk_args &, hipStream_t);

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
