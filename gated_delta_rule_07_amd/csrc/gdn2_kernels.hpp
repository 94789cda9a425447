// gdn2_kernels.hpp -- host-side declarations of the libgdn2 kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn2 {

typedef uint16_t bf16_t;  // raw bfloat16 bits

// Everything the chunked forward's kernels need.  All pointers are device
// pointers.  The workspace holds, for packed input, the per-sequence chunk
// offsets (offsets[n] = index of sequence n's first chunk, offsets[N] = total
// chunk count) followed by one block of per-chunk intermediates for every
// (chunk slot, head).
struct chunk_args {
  const void *q, *k, *v, *al, *b, *w;
  const float *S0;
  const int32_t *cu;  // packed sequence starts [N+1] or nullptr
  int32_t *offsets;   // [N+1] in the workspace (packed input only)
  int B, T, H, num_seqs, num_slots;
  void *o;
  float *S_final;
  char *blocks;      // num_slots * H blocks of blk_bytes each
  size_t blk_bytes;
  uint32_t gates;    // GATE_* bits: inputs given per (token, head) instead of per channel
  void *states;      // backward only: state entering every chunk (state_tiles blocks, slot * H + h)
  // Forward segment schedule: G > 0 when the call's sequences are segments,
  // seg_G consecutive ones per original sequence.  The segment map then
  // skips each sequence's last segment (no later segment needs its map),
  // and the state scan writes S_final only for that last segment, at the
  // original sequence's index.  0 otherwise.
  int seg_G;
};

// chunk_args::gates: b, w or alpha is one value per (token, head), laid out
// [B, T, H] (or [1, T_total, H] packed), shared by all of its channels.
// GATE_LAYER_PREP: the inputs are the raw layer inputs (q, k not normalised,
// b and w logits, alpha a float32 natural-log decay); the kernels apply the
// L2 norm, the sigmoid and exp themselves.
constexpr uint32_t GATE_SCALAR_B = 1u, GATE_SCALAR_W = 2u, GATE_SCALAR_ALPHA = 4u, GATE_LAYER_PREP = 8u;

template <typename IO, int D, int C> size_t chunk_block_bytes();
template <typename IO, int D, int C> hipError_t launch_chunk_prep(const chunk_args &a, hipStream_t st);
template <typename IO, int D, int C> hipError_t launch_chunk_scan(const chunk_args &a, hipStream_t st);
// the state scan in states mode: a.states instead of o (o is not written)
template <typename IO, int D, int C> hipError_t launch_chunk_states(const chunk_args &a, hipStream_t st);
// the forward scan that also writes the states-mode output (a.states): o,
// S_final and the state entering every chunk
template <typename IO, int D, int C> hipError_t launch_chunk_scan_keep(const chunk_args &a, hipStream_t st);
// rule R1's state scan on the scan kernel above (bfloat16, even numbers of
// 16-wide tiles in D and C; otherwise hipErrorNotSupported)
template <typename IO, int D, int C> constexpr bool scan_r1_supported() {
  return sizeof(IO) == 2 && (D / 16) % 2 == 0 && (C / 16) % 2 == 0;
}
template <typename IO, int D, int C> hipError_t launch_chunk_scan_r1(const chunk_args &a, hipStream_t st);
hipError_t launch_chunk_table(const int32_t *cu, int N, int C, int32_t *offsets, hipStream_t st);
// dst[u][r][c] (Rd x Cd per u) = src[u][r][c] where r < Rs and c < Cs, else
// the raw bits fill_bits; elements of elem_bytes (2 or 4) bytes
// (gdn2_pad.hip: widening for calls with dk != dv).
hipError_t launch_pad(const void *src, void *dst, long long U, int Rs, int Cs, int Rd, int Cd, int elem_bytes,
                      uint32_t fill_bits, hipStream_t st);
template <typename IO, int D, int C, int NG> bool fused_supported();
template <typename IO, int D, int C, int NG> hipError_t launch_fused(const chunk_args &a, hipStream_t st);

// Everything the chunked backward's own kernels need on top of the forward's
// arguments (inputs, chunk table, per-chunk blocks and entering states).
struct bwd_args {
  chunk_args f;
  const void *dout;      // dL/do [B, T, H, dv], element type IO
  const float *dSf;      // dL/dS_final [N, H, dk, dv] or nullptr (zero)
  void *dstates;         // dL/d(state leaving each chunk), state_tiles blocks like states
  float *dS0;            // dL/dS0 [N, H, dk, dv] or nullptr
  void *dq, *dk, *dv, *dal, *db, *dw;  // gradients, element type IO, input layouts
  unsigned char *pwflag;  // [num_slots * H]: chunk-heads whose gradients need the pairwise diagonal path
};

// Rule R1 on the two-pass path: its own per-chunk kernel and state scan, on
// blocks of r1_block_bytes (not instantiated for float32, D = 128, C = 64).
template <typename IO, int D, int C> size_t r1_block_bytes();
template <typename IO, int D, int C> hipError_t launch_r1_prep(const chunk_args &a, hipStream_t st);
template <typename IO, int D, int C> hipError_t launch_r1_scan(const chunk_args &a, hipStream_t st);

template <typename IO, int D, int C> hipError_t launch_bwd_dstate(const bwd_args &a, hipStream_t st);
template <typename IO, int D, int C> hipError_t launch_bwd_grad(const bwd_args &a, hipStream_t st);

// Affine state map of every sequence taken as one segment: Phi [N, H, D, D]
// and Psi [N, H, D, D] float32, row-major, from the prepared blocks.
template <typename IO, int D, int C> hipError_t launch_segmap(const chunk_args &a, float *Phi, float *Psi, hipStream_t st);
// seg_cu[0 .. B G] = the bounds of G segments of whole chunks (C tokens) of
// each of B sequences laid end to end: packed ones given by cu, else B
// sequences of T tokens (cu == nullptr).
// (offsets: also the segments' chunk table, [B G + 1], or nullptr)
hipError_t launch_seg_bounds(const int32_t *cu, int32_t *seg_cu, int G, int T, int B, int C, hipStream_t st,
                             int32_t *offsets = nullptr);
// Exclusive scan of the G segment maps of each of B sequences, [B, G, H, D, D],
// from S0 [B, H, D, D] (nullptr: zero).  reverse: the backward's adjoint
// scan (Phi transposed, segments from the last; see the kernel).
template <int D>
hipError_t launch_seg_combine(const float *Phi, const float *Psi, const float *S0, int G, int H, int B,
                              float *S_in, float *S_final, hipStream_t st, bool reverse = false);

template <typename IO, int DK, int DV>
hipError_t launch_decode(const void *q, const void *k, const void *v, const void *al,
                         const void *b, const void *w, float *S, void *o, int N, int H,
                         hipStream_t st);
template <typename IO, int DK, int DV>
hipError_t launch_recurrent(const void *q, const void *k, const void *v, const void *al,
                            const void *b, const void *w, const float *S0, const int32_t *cu,
                            int T, int H, int num_seqs, void *o, float *S_final, bool r1,
                            hipStream_t st);

}  // namespace gdn2
