// Entering states of the segments of a long sequence (dn_chunk_fwd_long).
//
// Over one segment the recurrence is affine in its entering state: the state
// after the segment is S_out = A S_in + B, A the product of the per-token
// maps (I - w_t k_t^T) D_t and B the end state reached from S_in = 0 (the
// affine memory scan of Kalman Delta Networks §2.6, Eq. 39, taken over a
// segment instead of a token).  The chunked forward computes every segment's
// A (from S_in = I with v = 0) and B (from S_in = 0) in parallel; this kernel
// chains them in order,
//   S_in(0) = S0,   S_in(s + 1) = A_s S_in(s) + B_s,   S_final = S_in(nseg),
// and the chunked forward then reruns every segment from its S_in.
//
// One workgroup per (batch, head, 32 value columns): the 32 columns of the
// running state sit in LDS, A_s is staged through LDS, and thread
// (row group rg, column group cg) forms 4 columns of DK / 32 rows in fp32.
#include "common.hpp"
#include "launch.hpp"

namespace dn {

constexpr int SC_THREADS = 256;
constexpr int SC_COLS = 32;  // value columns per workgroup

template <int DK>
__global__ __launch_bounds__(SC_THREADS) void segment_combine_kernel(CombineArgs a) {
  constexpr int CG = SC_COLS / 4;          // column groups of 4
  constexpr int RG = SC_THREADS / CG;      // row groups
  constexpr int RPT = DK / RG;             // rows per thread
  static_assert(RPT * RG == DK, "row split");
  // dynamic LDS: A_s [DK][DK + 4] (the pitch spreads the rows of a wavefront
  // over the banks), then the state [DK][SC_COLS]
  extern __shared__ __align__(16) float sc_smem[];
  float (*sA)[DK + 4] = reinterpret_cast<float (*)[DK + 4]>(sc_smem);
  float (*sX)[SC_COLS] = reinterpret_cast<float (*)[SC_COLS]>(sc_smem + DK * (DK + 4));

  const int tid = threadIdx.x;
  const int cg = tid % CG, rg = tid / CG;
  const int nsl = a.dv / SC_COLS;
  const long bh = blockIdx.x / nsl;
  const int col0 = (blockIdx.x % nsl) * SC_COLS + 4 * cg;

  // the state entering segment 0
  f32x4 x[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    x[i] = a.S0 ? *reinterpret_cast<const f32x4*>(&a.S0[(bh * DK + r) * a.dv + col0]) : zero4();
    *reinterpret_cast<f32x4*>(&sX[r][4 * cg]) = x[i];
  }
  for (int s = 0; s < a.nseg; ++s) {
    const long seg = bh * a.nseg + s;  // head index of the segment in the [B, H nseg] view
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *reinterpret_cast<f32x4*>(&a.S_in[(seg * DK + rg + RG * i) * a.dv + col0]) = x[i];
    // A_s through LDS, 16-byte rows
    const float* As = a.A + seg * DK * DK;
    for (int e = 4 * tid; e < DK * DK; e += 4 * SC_THREADS)
      *reinterpret_cast<f32x4*>(&sA[e / DK][e % DK]) = *reinterpret_cast<const f32x4*>(&As[e]);
    __syncthreads();  // A_s and the entering state visible
    // x <- A_s x + B_s
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + RG * i;
      f32x4 acc = *reinterpret_cast<const f32x4*>(&a.Bs[(seg * DK + r) * a.dv + col0]);
#pragma unroll 8
      for (int kk = 0; kk < DK; ++kk) {
        const float av = sA[r][kk];
        const f32x4 xv = *reinterpret_cast<const f32x4*>(&sX[kk][4 * cg]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = fmaf(av, xv[j], acc[j]);
      }
      x[i] = acc;
    }
    __syncthreads();  // every read of sA and sX done
#pragma unroll
    for (int i = 0; i < RPT; ++i) *reinterpret_cast<f32x4*>(&sX[rg + RG * i][4 * cg]) = x[i];
  }
  if (a.S_final) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *reinterpret_cast<f32x4*>(&a.S_final[(bh * DK + rg + RG * i) * a.dv + col0]) = x[i];
  }
}

template <int DK>
static hipError_t launch_sc(const CombineArgs& a, hipStream_t st) {
  const size_t smem = sizeof(float) * (DK * (DK + 4) + DK * SC_COLS);
  static_assert(sizeof(float) * (DK * (DK + 4) + DK * SC_COLS) <= 160 * 1024, "LDS budget");
  auto kern = segment_combine_kernel<DK>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (err != hipSuccess) return err;
  dim3 grid(static_cast<unsigned>(a.B * a.H * (a.dv / SC_COLS))), block(SC_THREADS);
  hipLaunchKernelGGL(kern, grid, block, smem, st, a);
  return hipGetLastError();
}

hipError_t launch_segment_combine(const CombineArgs& a, hipStream_t st) {
  return a.dk == 128 ? launch_sc<128>(a, st) : launch_sc<64>(a, st);
}

}  // namespace dn
