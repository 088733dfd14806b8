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
// One workgroup per (batch, head, 4 value columns): the 4 columns of the
// running state sit in LDS, A_s is staged through LDS (the next segment's A
// is loaded into registers while the current one is applied), and the KS =
// 256 / d_k adjacent lanes of row r each sum d_k / KS of the k terms of its 4
// columns in fp32, their partial sums then exchanged between the lanes.
#include "common.hpp"
#include "launch.hpp"

namespace dn {

constexpr int SC_THREADS = 256;
constexpr int SC_COLS = 4;

template <int DK>
__global__ __launch_bounds__(SC_THREADS) void segment_combine_kernel(CombineArgs a) {
  constexpr int KS = SC_THREADS / DK;              // lanes per row (k split)
  constexpr int KL = DK / KS;                      // k terms per lane
  constexpr int NA = DK * DK / (4 * SC_THREADS);   // 16-byte pieces of A per thread
  static_assert(KS * DK == SC_THREADS && (KS == 2 || KS == 4) && KL % 8 == 0, "work split");
  static_assert(NA * 4 * SC_THREADS == DK * DK, "A split");
  // dynamic LDS: A_s [DK][DK + 4] (the pitch spreads the rows of a wavefront
  // over the banks), then the state [DK][4]
  extern __shared__ __align__(16) float sc_smem[];
  DN_LDS_POISON(sc_smem, (DK * (DK + 4) + DK * SC_COLS) * sizeof(float));
  float (*sA)[DK + 4] = reinterpret_cast<float (*)[DK + 4]>(sc_smem);
  f32x4* sX = reinterpret_cast<f32x4*>(sc_smem + DK * (DK + 4));

  const int tid = threadIdx.x;
  const int ks = tid % KS, r = tid / KS;
  const int k0 = ks * KL;
  const int nsl = a.dv / SC_COLS;
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
  const int col0 = slice * SC_COLS;
  const bool lead = ks == 0;  // the lane of a row that stores it

  f32x4 an[NA];
  auto load_a = [&](long seg) {
    const float* As = a.A + seg * DK * DK;
#pragma unroll
    for (int j = 0; j < NA; ++j) an[j] = *reinterpret_cast<const f32x4*>(&As[4 * (tid + j * SC_THREADS)]);
  };
  // the state entering segment 0 (every lane of the row holds it)
  f32x4 x = a.S0 ? *reinterpret_cast<const f32x4*>(&a.S0[(bh * DK + r) * a.dv + col0]) : zero4();
  if (lead) sX[r] = x;
  load_a(bh * a.nseg);
  // B_s of the current segment, loaded one step ahead like A
  f32x4 bn = *reinterpret_cast<const f32x4*>(&a.Bs[(bh * a.nseg * DK + r) * a.dv + col0]);
  for (int s = 0; s < a.nseg; ++s) {
    const long seg = bh * a.nseg + s;  // head index of the segment in the [B, H nseg] view
    if (lead) *reinterpret_cast<f32x4*>(&a.S_in[(seg * DK + r) * a.dv + col0]) = x;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const int e = 4 * (tid + j * SC_THREADS);
      *reinterpret_cast<f32x4*>(&sA[e / DK][e % DK]) = an[j];
    }
    // the lane's partial sum starts from B_s on the row's first lane
    f32x4 xp = lead ? bn : zero4();
    if (s + 1 < a.nseg) {
      load_a(seg + 1);
      bn = *reinterpret_cast<const f32x4*>(&a.Bs[((seg + 1) * DK + r) * a.dv + col0]);
    }
    __syncthreads();  // A_s and the entering state visible
    // eight k per step: every read of a step is issued before its arithmetic
#pragma unroll 2
    for (int kk = k0; kk < k0 + KL; kk += 8) {
      f32x4 a8[2], xv[8];
#pragma unroll
      for (int h = 0; h < 2; ++h) a8[h] = *reinterpret_cast<const f32x4*>(&sA[r][kk + 4 * h]);
#pragma unroll
      for (int q = 0; q < 8; ++q) xv[q] = sX[kk + q];
#pragma unroll
      for (int q = 0; q < 8; ++q)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) xp[jj] = fmaf(a8[q / 4][q % 4], xv[q][jj], xp[jj]);
    }
    // sum over the row's lanes (adjacent lanes of one wavefront); the lanes'
    // additions differ only by commutation, so all of them hold the same x
#pragma unroll
    for (int m = 1; m < KS; m *= 2)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) xp[jj] += __shfl_xor(xp[jj], m);
    x = xp;
    __syncthreads();  // every read of sA and sX done
    if (lead) sX[r] = x;
  }
  // a head the chunk form could not evaluate keeps S0 (S_final may be S0):
  // the tokenwise pass writes its final state
  bool oor = false;
  if (a.oor)
    for (int s = 0; s < a.nseg; ++s) oor |= a.oor[bh * a.nseg + s] != 0;
  if (a.S_final && lead && !oor) *reinterpret_cast<f32x4*>(&a.S_final[(bh * DK + r) * a.dv + col0]) = x;
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
