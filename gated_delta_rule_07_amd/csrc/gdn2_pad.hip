// gdn2_pad.hip -- copies between rectangular and square layouts, for calls
// whose key and value widths differ (dk != dv).
//
// The chunked kernels are built for square heads (dk = dv = d).  A call with
// dk != dv runs on d = max(dk, dv) with the narrower side widened by
// channels that cannot reach the result: widened key channels carry
// q = k = b = 0 and no decay (alpha = 1, log-decay 0), so their state rows
// stay at zero and add nothing to o = S^T q; widened value channels carry
// v = w = 0, so their state columns stay at zero and their outputs are
// dropped.  This file moves tensors into and out of the widened layout.
#include "gdn2_kernels.hpp"

namespace gdn2 {

// dst[u][r][c] (Rd x Cd per u) = src[u][r][c] where r < Rs and c < Cs, else
// `fill`.  Elements of E bytes (2 or 4), moved as raw bits.  One thread per
// destination element, grid-stride.
template <typename E>
__global__ void __launch_bounds__(256)
    gdn2_pad_kernel(const E *__restrict__ src, E *__restrict__ dst, long long U, int Rs, int Cs, int Rd, int Cd,
                    E fill) {
  const long long per = static_cast<long long>(Rd) * Cd;
  const long long total = U * per;
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  for (long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += stride) {
    const long long u = i / per;
    const int rc = static_cast<int>(i - u * per);
    const int r = rc / Cd, c = rc - r * Cd;
    dst[i] = (r < Rs && c < Cs) ? src[(u * Rs + r) * Cs + c] : fill;
  }
}

hipError_t launch_pad(const void *src, void *dst, long long U, int Rs, int Cs, int Rd, int Cd, int elem_bytes,
                      uint32_t fill_bits, hipStream_t st) {
  const long long total = U * Rd * Cd;
  if (total <= 0)
    return hipSuccess;
  const long long want = (total + 255) / 256;
  const unsigned blocks = static_cast<unsigned>(want < 8192 ? want : 8192);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(gdn2_pad_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st, static_cast<const uint16_t *>(src),
                       static_cast<uint16_t *>(dst), U, Rs, Cs, Rd, Cd, static_cast<uint16_t>(fill_bits));
  else if (elem_bytes == 4)
    hipLaunchKernelGGL(gdn2_pad_kernel<uint32_t>, dim3(blocks), dim3(256), 0, st, static_cast<const uint32_t *>(src),
                       static_cast<uint32_t *>(dst), U, Rs, Cs, Rd, Cd, fill_bits);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace gdn2
