// gdn2_recurrent.hip -- token-at-a-time GDN-2 kernels for gfx950:
//   gdn2_decode_kernel    one decode step for every (sequence, head), state in
//                         HBM updated in place (the constant-memory decode of
//                         the aixai.ru blog and needhelp.icu/de pages);
//   gdn2_recurrent_kernel the same update looped over whole sequences with the
//                         state held in registers (a slow, simple cross-check
//                         of the chunked kernels).
//
// Per token, for one head (S is dk x dv, row = key channel):
//   r_j = sum_i alpha_i b_i k_i S_ij
//   S_ij <- alpha_i S_ij + k_i (w_j v_j - r_j)
//   o_j = sum_i q_i S_ij            (after the update)
// which is D = Diag(alpha) S, z = w (.) v - D^T (b (.) k), S = D + k z^T,
// o = S^T q (aixai.ru blog, formal paragraph of the gate section).
//
// The recurrent kernel also runs the alternative reading R1, in which b only
// places the erase and the read uses the plain key:
//   r = D^T k;  S = D - (b (.) k) r^T + k (w (.) v)^T;  o = S^T q
// (the "location-gated erase": the same pages, read with the erase gate on
// the erased direction instead of on the read).
//
// Work split: one workgroup per (sequence, head).  A thread owns 4
// consecutive value columns in DK / ROWS_PER_PASS rows, so every state load
// and store is a 16-byte vector and a row of 4*DV/4 threads reads one
// contiguous row of S.  Column sums over rows go through LDS.
#include "gdn2_device.hpp"
#include "gdn2_kernels.hpp"

namespace gdn2 {

template <int DK, int DV> struct rec_shape {
  static constexpr int TPR = DV / 4;                              // threads per row
  static constexpr int NT = (TPR * DK < 256) ? TPR * DK : 256;    // threads
  static constexpr int RPP = NT / TPR;                            // rows per pass
  static constexpr int PASSES = DK / RPP;
  static_assert(DK % RPP == 0, "row split");
};

// Shared-memory staging of one token's vectors (float32).
template <int DK, int DV> struct rec_smem {
  float a[DK], e[DK], k[DK], q[DK];  // alpha, b*k, k, q
  float u[DV];                       // w*v
  float red[rec_shape<DK, DV>::RPP][DV];
  float z[DV];
};

template <typename IO, int DK, int DV>
__device__ __forceinline__ void rec_stage_token(rec_smem<DK, DV> &sm, const IO *q, const IO *k,
                                                const IO *v, const IO *al, const IO *b,
                                                const IO *w, int tid) {
  constexpr int NT = rec_shape<DK, DV>::NT;
  for (int i = tid; i < DK; i += NT) {
    const float kk = io<IO>::to_f(k[i]);
    sm.a[i] = io<IO>::to_f(al[i]);
    sm.e[i] = io<IO>::to_f(b[i]) * kk;
    sm.k[i] = kk;
    sm.q[i] = io<IO>::to_f(q[i]);
  }
  for (int j = tid; j < DV; j += NT)
    sm.u[j] = io<IO>::to_f(w[j]) * io<IO>::to_f(v[j]);
}

// One token update of the thread's state slice s[p] (rows tr + RPP*p,
// columns 4*tc .. 4*tc+3).  Writes o (DV values, element type IO) if o != 0.
// R1 selects the alternative reading above.
template <typename IO, int DK, int DV, bool R1 = false>
__device__ __forceinline__ void rec_token_update(rec_smem<DK, DV> &sm,
                                                 f32x4 (&s)[rec_shape<DK, DV>::PASSES], IO *o,
                                                 int tid) {
  typedef rec_shape<DK, DV> R;
  const int tc = tid % R::TPR, tr = tid / R::TPR;
  // read with the erase-gated key (R1: the plain key), from the decayed state
  f32x4 r = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < R::PASSES; ++p) {
    const int i = tr + R::RPP * p;
    s[p] *= sm.a[i];
    r += (R1 ? sm.k[i] : sm.e[i]) * s[p];
  }
  *reinterpret_cast<f32x4 *>(&sm.red[tr][4 * tc]) = r;
  __syncthreads();
  for (int j = tid; j < DV; j += R::NT) {
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < R::RPP; ++t)
      acc += sm.red[t][j];
    sm.z[j] = R1 ? acc : sm.u[j] - acc;  // R1 keeps the read r itself
  }
  __syncthreads();
  const f32x4 z = *reinterpret_cast<const f32x4 *>(&sm.z[4 * tc]);
  const f32x4 u4 = *reinterpret_cast<const f32x4 *>(&sm.u[4 * tc]);
  f32x4 oq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < R::PASSES; ++p) {
    const int i = tr + R::RPP * p;
    if constexpr (R1)
      s[p] += sm.k[i] * u4 - sm.e[i] * z;  // erase along b (.) k, write along k
    else
      s[p] += sm.k[i] * z;
    oq += sm.q[i] * s[p];
  }
  *reinterpret_cast<f32x4 *>(&sm.red[tr][4 * tc]) = oq;
  __syncthreads();
  if (o) {
    for (int j = tid; j < DV; j += R::NT) {
      float acc = 0.f;
#pragma unroll
      for (int t = 0; t < R::RPP; ++t)
        acc += sm.red[t][j];
      o[j] = io<IO>::from_f(acc);
    }
  }
  __syncthreads();
}

// grid: N*H workgroups; block: rec_shape::NT threads.  STREAM: the state is
// read and written with nontemporal hints (no allocation in the caches on
// the way), for states too large to stay cache-resident between steps.
template <typename IO, int DK, int DV, bool STREAM>
__global__ void __launch_bounds__((rec_shape<DK, DV>::NT))
    gdn2_decode_kernel(const IO *__restrict__ q, const IO *__restrict__ k,
                       const IO *__restrict__ v, const IO *__restrict__ al,
                       const IO *__restrict__ b, const IO *__restrict__ w, float *S, IO *o,
                       int units) {
  typedef rec_shape<DK, DV> R;
  __shared__ rec_smem<DK, DV> sm;
  const int u = blockIdx.x;
  if (u >= units)
    return;
  const int tid = threadIdx.x;
  const int tc = tid % R::TPR, tr = tid / R::TPR;
  float *Su = S + static_cast<size_t>(u) * DK * DV;
  f32x4 s[R::PASSES];
#pragma unroll
  for (int p = 0; p < R::PASSES; ++p) {
    const f32x4 *src = reinterpret_cast<const f32x4 *>(Su + (tr + R::RPP * p) * DV + 4 * tc);
    s[p] = STREAM ? __builtin_nontemporal_load(src) : *src;
  }
  rec_stage_token<IO, DK, DV>(sm, q + static_cast<size_t>(u) * DK, k + static_cast<size_t>(u) * DK,
                              v + static_cast<size_t>(u) * DV, al + static_cast<size_t>(u) * DK,
                              b + static_cast<size_t>(u) * DK, w + static_cast<size_t>(u) * DV, tid);
  __syncthreads();
  rec_token_update<IO, DK, DV>(sm, s, o + static_cast<size_t>(u) * DV, tid);
#pragma unroll
  for (int p = 0; p < R::PASSES; ++p) {
    f32x4 *dst = reinterpret_cast<f32x4 *>(Su + (tr + R::RPP * p) * DV + 4 * tc);
    if constexpr (STREAM)
      __builtin_nontemporal_store(s[p], dst);
    else
      *dst = s[p];
  }
}

// grid: N*H workgroups (unit = n*H + h); block: rec_shape::NT threads.
// Fixed length when cu == nullptr (sequence n = batch row n of length T).
template <typename IO, int DK, int DV, bool R1>
__global__ void __launch_bounds__((rec_shape<DK, DV>::NT))
    gdn2_recurrent_kernel(const IO *__restrict__ q, const IO *__restrict__ k,
                          const IO *__restrict__ v, const IO *__restrict__ al,
                          const IO *__restrict__ b, const IO *__restrict__ w,
                          const float *S0, const int32_t *__restrict__ cu, int T, int H,
                          int num_seqs, IO *__restrict__ o, float *S_final) {
  typedef rec_shape<DK, DV> R;
  __shared__ rec_smem<DK, DV> sm;
  const int u = blockIdx.x;
  if (u >= num_seqs * H)
    return;
  const int n = u / H, h = u % H;
  const int tid = threadIdx.x;
  const int tc = tid % R::TPR, tr = tid / R::TPR;
  f32x4 s[R::PASSES];
  if (S0) {
    const float *Su = S0 + static_cast<size_t>(u) * DK * DV;
#pragma unroll
    for (int p = 0; p < R::PASSES; ++p)
      s[p] = *reinterpret_cast<const f32x4 *>(Su + (tr + R::RPP * p) * DV + 4 * tc);
  } else {
#pragma unroll
    for (int p = 0; p < R::PASSES; ++p)
      s[p] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  long t0, t1;
  if (cu) {
    t0 = cu[n];
    t1 = cu[n + 1];
  } else {
    t0 = static_cast<long>(n) * T;
    t1 = t0 + T;
  }
  for (long t = t0; t < t1; ++t) {
    const size_t row = static_cast<size_t>(t) * H + h;
    rec_stage_token<IO, DK, DV>(sm, q + row * DK, k + row * DK, v + row * DV, al + row * DK,
                                b + row * DK, w + row * DV, tid);
    __syncthreads();
    rec_token_update<IO, DK, DV, R1>(sm, s, o + row * DV, tid);
  }
  if (S_final) {
    float *Su = S_final + static_cast<size_t>(u) * DK * DV;
#pragma unroll
    for (int p = 0; p < R::PASSES; ++p)
      *reinterpret_cast<f32x4 *>(Su + (tr + R::RPP * p) * DV + 4 * tc) = s[p];
  }
}

// ------------------------------------------------------------- launchers --
template <typename IO, int DK, int DV>
hipError_t launch_decode(const void *q, const void *k, const void *v, const void *al,
                         const void *b, const void *w, float *S, void *o, int N, int H,
                         hipStream_t st) {
  typedef rec_shape<DK, DV> R;
  const int units = N * H;
  // A state of 64 MiB or more is streamed: in a model's decode loop the
  // layers' states take turns, so one this large is never cache-resident
  // when its layer comes round again, and the hints let the reads and
  // writes run at streaming rate (256 x 16 heads, d = 128, 256 MiB: 94.9 us
  // per step against 107.3 us when another state of that size ran in
  // between, but 80.4 us cached when the same state is stepped back to
  // back).
  const bool stream = static_cast<size_t>(units) * DK * DV * sizeof(float) >= (static_cast<size_t>(64) << 20);
  if (stream)
    hipLaunchKernelGGL((gdn2_decode_kernel<IO, DK, DV, true>), dim3(units), dim3(R::NT), 0, st,
                       static_cast<const IO *>(q), static_cast<const IO *>(k), static_cast<const IO *>(v),
                       static_cast<const IO *>(al), static_cast<const IO *>(b), static_cast<const IO *>(w), S,
                       static_cast<IO *>(o), units);
  else
    hipLaunchKernelGGL((gdn2_decode_kernel<IO, DK, DV, false>), dim3(units), dim3(R::NT), 0, st,
                       static_cast<const IO *>(q), static_cast<const IO *>(k), static_cast<const IO *>(v),
                       static_cast<const IO *>(al), static_cast<const IO *>(b), static_cast<const IO *>(w), S,
                       static_cast<IO *>(o), units);
  return hipGetLastError();
}

template <typename IO, int DK, int DV>
hipError_t launch_recurrent(const void *q, const void *k, const void *v, const void *al,
                            const void *b, const void *w, const float *S0, const int32_t *cu,
                            int T, int H, int num_seqs, void *o, float *S_final, bool r1,
                            hipStream_t st) {
  typedef rec_shape<DK, DV> R;
  if (r1)
    hipLaunchKernelGGL((gdn2_recurrent_kernel<IO, DK, DV, true>), dim3(num_seqs * H), dim3(R::NT), 0, st,
                       static_cast<const IO *>(q), static_cast<const IO *>(k),
                       static_cast<const IO *>(v), static_cast<const IO *>(al),
                       static_cast<const IO *>(b), static_cast<const IO *>(w), S0, cu, T, H,
                       num_seqs, static_cast<IO *>(o), S_final);
  else
    hipLaunchKernelGGL((gdn2_recurrent_kernel<IO, DK, DV, false>), dim3(num_seqs * H), dim3(R::NT), 0, st,
                       static_cast<const IO *>(q), static_cast<const IO *>(k),
                       static_cast<const IO *>(v), static_cast<const IO *>(al),
                       static_cast<const IO *>(b), static_cast<const IO *>(w), S0, cu, T, H,
                       num_seqs, static_cast<IO *>(o), S_final);
  return hipGetLastError();
}

// every (dk, dv) pair of {16, 32, 64, 128}: the state is dk x dv
#define GDN2_INST_REC(IO, DK, DV)                                                              \
  template hipError_t launch_decode<IO, DK, DV>(const void *, const void *, const void *,    \
                                                const void *, const void *, const void *,     \
                                                float *, void *, int, int, hipStream_t);       \
  template hipError_t launch_recurrent<IO, DK, DV>(                                           \
      const void *, const void *, const void *, const void *, const void *, const void *,     \
      const float *, const int32_t *, int, int, int, void *, float *, bool, hipStream_t);
#define GDN2_INST_REC_DK(IO, DK) \
  GDN2_INST_REC(IO, DK, 16) GDN2_INST_REC(IO, DK, 32) GDN2_INST_REC(IO, DK, 64) GDN2_INST_REC(IO, DK, 128)

GDN2_INST_REC_DK(float, 16)
GDN2_INST_REC_DK(float, 32)
GDN2_INST_REC_DK(float, 64)
GDN2_INST_REC_DK(float, 128)
GDN2_INST_REC_DK(bf16_t, 16)
GDN2_INST_REC_DK(bf16_t, 32)
GDN2_INST_REC_DK(bf16_t, 64)
GDN2_INST_REC_DK(bf16_t, 128)

}  // namespace gdn2
