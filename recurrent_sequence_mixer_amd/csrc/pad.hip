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
// Each thread moves one 16-byte piece of a destination row (cs and cd are
// multiples of the piece, rows start on 16-byte boundaries).
template <typename E>
__global__ void reshape3_kernel(const E* src, E* dst, long outer, int rs, int cs, int rd, int cd,
                                E fill) {
  constexpr int VE = 16 / sizeof(E);  // elements per piece
  const int pr = cd / VE;             // pieces per destination row
  const long rows = outer * rd, n = rows * pr;
  E fv[VE];
#pragma unroll
  for (int i = 0; i < VE; ++i) fv[i] = fill;
  const u32x4 fill4 = *reinterpret_cast<const u32x4*>(fv);
  for (long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<long>(gridDim.x) * blockDim.x) {
    const long row = i / pr;
    const int c = static_cast<int>(i - row * pr) * VE;
    const long o = row / rd;
    const int r = static_cast<int>(row - o * rd);
    u32x4 x = fill4;
    if (r < rs && c < cs) x = *reinterpret_cast<const u32x4*>(src + (o * rs + r) * cs + c);
    *reinterpret_cast<u32x4*>(dst + row * cd + c) = x;
  }
}

hipError_t launch_reshape3(const void* src, void* dst, long outer, int rs, int cs, int rd, int cd,
                           int esize, uint32_t fill_bits, hipStream_t st) {
  const int ve = 16 / esize;
  if (cs % ve != 0 || cd % ve != 0) return hipErrorInvalidValue;
  const long n = outer * rd * (cd / ve);
  if (n == 0) return hipSuccess;
  const long blocks = (n + 255) / 256;
  const dim3 grid(static_cast<unsigned>(blocks < 16384 ? blocks : 16384)), block(256);
  if (esize == 2)
    hipLaunchKernelGGL(reshape3_kernel<uint16_t>, grid, block, 0, st, static_cast<const uint16_t*>(src),
                       static_cast<uint16_t*>(dst), outer, rs, cs, rd, cd, static_cast<uint16_t>(fill_bits));
  else
    hipLaunchKernelGGL(reshape3_kernel<float>, grid, block, 0, st, static_cast<const float*>(src),
                       static_cast<float*>(dst), outer, rs, cs, rd, cd, __builtin_bit_cast(float, fill_bits));
  return hipGetLastError();
}

}  // namespace dn
