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
// One workgroup per (batch, head, 4 x 256 / d_k value columns, 8 at d_k = 128): the columns of the
// running state sit in LDS, A_s is staged through LDS (the next segment's A
// is loaded into registers while the current one is applied), and thread
// (row r, column group cg) forms 4 columns of row r in fp32.
#include "common.hpp"
#include "launch.hpp"

namespace dn {

constexpr int SC_THREADS = 256;
template <int DK>
constexpr int sc_cols() { return 4 * SC_THREADS / DK; }  // one row per thread

template <int DK>
__global__ __launch_bounds__(SC_THREADS) void segment_combine_kernel(CombineArgs a) {
  constexpr int COLS = sc_cols<DK>();
  constexpr int CG = COLS / 4;                      // column groups of 4
  constexpr int NA = DK * DK / (4 * SC_THREADS);    // 16-byte pieces of A per thread
  static_assert(CG * DK == SC_THREADS && NA * 4 * SC_THREADS == DK * DK, "work split");
  // dynamic LDS: A_s [DK][DK + 4] (the pitch spreads the rows of a wavefront
  // over the banks), then the state [DK][COLS]
  extern __shared__ __align__(16) float sc_smem[];
  float (*sA)[DK + 4] = reinterpret_cast<float (*)[DK + 4]>(sc_smem);
  float (*sX)[COLS] = reinterpret_cast<float (*)[COLS]>(sc_smem + DK * (DK + 4));

  const int tid = threadIdx.x;
  const int cg = tid % CG, r = tid / CG;
  const int nsl = a.dv / COLS;
  // XCD-aware mapping: consecutive workgroups are dealt to the 8 XCDs in turn;
  // every column slice of a head gets an id of the same residue modulo 8, so
  // that A_s comes into one XCD's L2 and is read there by all of them
  const int nwg = a.B * a.H * nsl;
  long bh;
  int slice;
  if (nwg % 8 == 0 && (nwg / 8) % nsl == 0) {
    const int xcd = blockIdx.x % 8, rr = blockIdx.x / 8;
    slice = rr % nsl;
    bh = static_cast<long>(xcd) * (nwg / 8 / nsl) + rr / nsl;
  } else {
    slice = blockIdx.x % nsl;
    bh = blockIdx.x / nsl;
  }
  const int col0 = slice * COLS + 4 * cg;

  f32x4 an[NA];
  auto load_a = [&](long seg) {
    const float* As = a.A + seg * DK * DK;
#pragma unroll
    for (int j = 0; j < NA; ++j) an[j] = *reinterpret_cast<const f32x4*>(&As[4 * (tid + j * SC_THREADS)]);
  };
  // the state entering segment 0
  f32x4 x = a.S0 ? *reinterpret_cast<const f32x4*>(&a.S0[(bh * DK + r) * a.dv + col0]) : zero4();
  *reinterpret_cast<f32x4*>(&sX[r][4 * cg]) = x;
  load_a(bh * a.nseg);
  // B_s of the current segment, loaded one step ahead like A
  f32x4 bn = *reinterpret_cast<const f32x4*>(&a.Bs[(bh * a.nseg * DK + r) * a.dv + col0]);
  for (int s = 0; s < a.nseg; ++s) {
    const long seg = bh * a.nseg + s;  // head index of the segment in the [B, H nseg] view
    *reinterpret_cast<f32x4*>(&a.S_in[(seg * DK + r) * a.dv + col0]) = x;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int e = 4 * (tid + j * SC_THREADS);
      *reinterpret_cast<f32x4*>(&sA[e / DK][e % DK]) = an[j];
    }
    x = bn;
    if (s + 1 < a.nseg) {
      load_a(seg + 1);
      bn = *reinterpret_cast<const f32x4*>(&a.Bs[((seg + 1) * DK + r) * a.dv + col0]);
    }
    __syncthreads();  // A_s and the entering state visible
    // x <- A_s x + B_s: eight k per step, A read as 16-byte pieces of row r;
    // every read of a step is issued before its arithmetic, so that the LDS
    // latency is paid once per eight k rather than once per k
#pragma unroll 2
    for (int kk = 0; kk < DK; kk += 8) {
      f32x4 a8[2], xv[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) a8[h] = *reinterpret_cast<const f32x4*>(&sA[r][kk + 4 * h]);
#pragma unroll
      for (int q = 0; q < 8; ++q) xv[q] = *reinterpret_cast<const f32x4*>(&sX[kk + q][4 * cg]);
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) x[jj] = fmaf(a8[q / 4][q % 4], xv[q][jj], x[jj]);
    }
    __syncthreads();  // every read of sA and sX done
    *reinterpret_cast<f32x4*>(&sX[r][4 * cg]) = x;
  }
  if (a.S_final) *reinterpret_cast<f32x4*>(&a.S_final[(bh * DK + r) * a.dv + col0]) = x;
}

template <int DK>
static hipError_t launch_sc(const CombineArgs& a, hipStream_t st) {
  constexpr int COLS = sc_cols<DK>();
  const size_t smem = sizeof(float) * (DK * (DK + 4) + DK * COLS);
  static_assert(sizeof(float) * (DK * (DK + 4) + DK * COLS) <= 160 * 1024, "LDS budget");
  auto kern = segment_combine_kernel<DK>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(smem));
  if (err != hipSuccess) return err;
  dim3 grid(static_cast<unsigned>(a.B * a.H * (a.dv / COLS))), block(SC_THREADS);
  hipLaunchKernelGGL(kern, grid, block, smem, st, a);
  return hipGetLastError();
}

hipError_t launch_segment_combine(const CombineArgs& a, hipStream_t st) {
  return a.dk == 128 ? launch_sc<128>(a, st) : launch_sc<64>(a, st);
}

}  // namespace dn
