// Copies between a tensor of head width (d_k or d_v) that no kernel is built
// for and the same tensor at the next kernel width, padded.  Head widths that
// are multiples of 8 up to 128 (the 120-wide heads of the 1B architecture of
// Preconditioned DeltaNet §3.1, for example) run on the 64- or 128-wide
// kernels: every padded key channel has k = q = w = 0 and decay 1, every
// padded value column v = 0, so the recurrence restricted to the real
// channels and columns is the one of the unpadded head, and the padded state
// rows and columns stay 0.
#include "common.hpp"
#include "launch.hpp"

namespace dn {

// dst[o][r][c] = src[o][r][c] where r < rs and c < cs, else fill; for
// r < rd, c < cd (src is [outer][rs][cs], dst [outer][rd][cd]).  Serves both
// directions: padding (rd >= rs, cd >= cs) and cropping (rd <= rs, cd <= cs).
template <typename E>
__global__ void reshape3_kernel(const E* src, E* dst, long outer, int rs, int cs, int rd, int cd,
                                E fill) {
  const long n = outer * rd * cd;
  for (long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<long>(gridDim.x) * blockDim.x) {
    const int c = static_cast<int>(i % cd);
    const long t = i / cd;
    const int r = static_cast<int>(t % rd);
    const long o = t / rd;
    dst[i] = r < rs && c < cs ? src[(o * rs + r) * cs + c] : fill;
  }
}

hipError_t launch_reshape3(const void* src, void* dst, long outer, int rs, int cs, int rd, int cd,
                           int esize, uint32_t fill_bits, hipStream_t st) {
  const long n = outer * rd * cd;
  if (n == 0) return hipSuccess;
  const long blocks = (n + 255) / 256;
  const dim3 grid(static_cast<unsigned>(blocks < 8192 ? blocks : 8192)), block(256);
  if (esize == 2)
    hipLaunchKernelGGL(reshape3_kernel<uint16_t>, grid, block, 0, st, static_cast<const uint16_t*>(src),
                       static_cast<uint16_t*>(dst), outer, rs, cs, rd, cd, static_cast<uint16_t>(fill_bits));
  else
    hipLaunchKernelGGL(reshape3_kernel<float>, grid, block, 0, st, static_cast<const float*>(src),
                       static_cast<float*>(dst), outer, rs, cs, rd, cd, __builtin_bit_cast(float, fill_bits));
  return hipGetLastError();
}

}  // namespace dn
