// Gain statistics entering the segments of a long sequence (dn_chunk_fwd_long).
//
// The write gains of PGDN and of diagonal and isotropic KDN carry a
// statistic from token to token that does not depend on the memory state S:
//   PGDN   A_t = alphaP_t A_{t-1} + betaP_t k_t^2, per key channel
//          (Preconditioned DeltaNet §2.4, Eq. 9): an affine map of A_{t-1};
//   KDN    p_t = p_hat / (1 + u p_hat), p_hat = alpha^2 p_{t-1} + omega,
//          u = mu k^2 / r, per key channel (Kalman Delta Networks §2.4-2.5):
//          the Moebius map with matrix [[1, 0], [u, 1]] [[alpha^2, omega], [0, 1]];
//   isotropic KDN: the same map on one scalar per head, with alpha^2 the mean
//          over the channels and u = mu ||k||^2 / (d_k r) (§2.7, Eq. 40).
// Maps of this kind compose (the associative gain scan of Kalman Delta
// Networks §2.6), so the statistic at every segment start comes from
// (1) segment_summary_kernel: the composed map of every piece of `lsub`
//     tokens, all pieces in parallel;
// (2) segment_chain_kernel: per head and channel, the pieces applied in order
//     from aux0, the value at each segment start written for the segment's
//     head of the [B, H nseg] view, and the value after the last token as
//     aux_final.
// A summary holds three floats per channel: PGDN (m, c, -) with
// A -> m A + c; KDN (m00, m01, m10) with p -> (m00 p + m01) / (m10 p + 1), the
// map's matrix kept normalised to a (1, 1) entry of 1 after every token.
#include "common.hpp"
#include "gains.hpp"
#include "launch.hpp"

namespace dn {

// One token of a Moebius summary: M <- [[1, 0], [u, 1]] [[a, om], [0, 1]] M,
// renormalised so that M(1, 1) = 1 (it is >= 1 before that, every entry being
// nonnegative).
__device__ __forceinline__ void mobius_step(float& m00, float& m01, float& m10, float a, float om,
                                            float u) {
  const float n00 = fmaf(a, m00, om * m10);
  const float n01 = fmaf(a, m01, om);
  const float n10 = fmaf(u, n00, m10);
  const float inv = 1.f / fmaf(u, n01, 1.f);
  m00 = n00 * inv;
  m01 = n01 * inv;
  m10 = n10 * inv;
}

// PGDN and diagonal KDN: one thread per key channel, one workgroup per piece.
// The loads of U tokens are issued before their arithmetic (the composition
// is a serial chain per channel; its inputs are not).
template <int DK, int GAIN>
__global__ __launch_bounds__(DK) void segment_summary_kernel(StatArgs a) {
  constexpr int U = 16;  // lsub is a multiple of 64
  const int c = threadIdx.x;
  const int nsub = a.T / a.lsub;
  const long bh = blockIdx.x / nsub;
  const long t0 = bh * a.T + static_cast<long>(blockIdx.x % nsub) * a.lsub;
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + t0 * DK + c;
  float s0, s1, s2;
  if constexpr (GAIN == GAIN_PGDN) {
    float m = 1.f, cc = 0.f;
    for (int i0 = 0; i0 < a.lsub; i0 += U) {
      float kk[U], ap[U], bp[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        kk[j] = bf2f(kp[static_cast<long>(i0 + j) * DK]);
        ap[j] = a.g.alphaP[t0 + i0 + j];
        bp[j] = a.g.betaP[t0 + i0 + j];
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        m *= ap[j];
        cc = fmaf(ap[j], cc, bp[j] * kk[j] * kk[j]);
      }
    }
    s0 = m, s1 = cc, s2 = 0.f;
  } else {
    const uint16_t* al = static_cast<const uint16_t*>(a.g.alpha) + t0 * DK + c;
    const uint16_t* om = static_cast<const uint16_t*>(a.g.omega) + t0 * DK + c;
    float m00 = 1.f, m01 = 0.f, m10 = 0.f;
    for (int i0 = 0; i0 < a.lsub; i0 += U) {
      float kk[U], aa[U], ww[U], rr[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const long o = static_cast<long>(i0 + j) * DK;
        kk[j] = bf2f(kp[o]);
        aa[j] = bf2f(al[o]);
        ww[j] = bf2f(om[o]);
        rr[j] = a.g.r[t0 + i0 + j];
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const float u = a.g.mu_info * kk[j] * kk[j] / rr[j];
        mobius_step(m00, m01, m10, aa[j] * aa[j], ww[j], u);
      }
    }
    s0 = m00, s1 = m01, s2 = m10;
  }
  float* out = a.summ + static_cast<long>(blockIdx.x) * 3 * DK + c;
  out[0] = s0;
  out[DK] = s1;
  out[2 * DK] = s2;
}

// Isotropic KDN: thread i forms token i's map from its channel sums; the
// piece's maps are then composed pairwise in a tree (later map on the left),
// every product renormalised to a (1, 1) entry of 1.  lsub is a power of two.
template <int DK>
__global__ __launch_bounds__(256) void segment_summary_iso_kernel(StatArgs a) {
  __shared__ float f00[256], f01[256], f10[256];
  const int i = threadIdx.x;
  const int nsub = a.T / a.lsub;
  const long bh = blockIdx.x / nsub;
  const long t0 = bh * a.T + static_cast<long>(blockIdx.x % nsub) * a.lsub;
  if (i < a.lsub) {
    const uint4* kr = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + (t0 + i) * DK);
    const uint4* ar = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.g.alpha) + (t0 + i) * DK);
    float nk = 0.f, sa = 0.f;
#pragma unroll 4
    for (int j = 0; j < DK / 8; ++j) {
      const uint4 kv = kr[j], av = ar[j];
      const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w}, aw[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float k0 = __uint_as_float(kw[e] << 16), k1 = __uint_as_float(kw[e] & 0xffff0000u);
        const float a0 = __uint_as_float(aw[e] << 16), a1 = __uint_as_float(aw[e] & 0xffff0000u);
        nk = fmaf(k0, k0, fmaf(k1, k1, nk));
        sa = fmaf(a0, a0, fmaf(a1, a1, sa));
      }
    }
    const float r = a.g.r[t0 + i];
    const float am = sa * (1.f / DK), om = static_cast<const float*>(a.g.omega)[t0 + i];
    const float u = a.g.mu_info * nk / (DK * r);
    // the token's map [[am, om], [u am, 1 + u om]] / (1 + u om)
    const float inv = 1.f / fmaf(u, om, 1.f);
    f00[i] = am * inv;
    f01[i] = om * inv;
    f10[i] = u * am * inv;
  }
  for (int w = 1; w < a.lsub; w *= 2) {
    __syncthreads();
    if (i % (2 * w) == 0 && i + w < a.lsub) {
      const float l00 = f00[i + w], l01 = f01[i + w], l10 = f10[i + w];
      const float r00 = f00[i], r01 = f01[i], r10 = f10[i];
      const float inv = 1.f / fmaf(l10, r01, 1.f);
      f00[i] = fmaf(l00, r00, l01 * r10) * inv;
      f01[i] = fmaf(l00, r01, l01) * inv;
      f10[i] = fmaf(l10, r00, r10) * inv;
    }
  }
  if (i == 0) {
    float* out = a.summ + static_cast<long>(blockIdx.x) * 3;
    out[0] = f00[0];
    out[1] = f01[0];
    out[2] = f10[0];
  }
}

// One thread per (head, channel): the pieces applied in order, their
// summaries loaded U at a time ahead of the serial arithmetic.
__global__ __launch_bounds__(64) void segment_chain_kernel(StatArgs a) {
  constexpr int U = 8;
  const int aph = a.gain == GAIN_KDN_ISO ? 1 : a.dk;
  const long item = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const long nitems = static_cast<long>(a.B) * a.H * aph;
  if (item < nitems) {
    const long bh = item / aph;
    const int c = static_cast<int>(item % aph);
    const int nsub = a.T / a.lsub, per = nsub / a.nseg;
    float x = a.aux0 ? a.aux0[item] : 1.f;
    const float* sm = a.summ + bh * nsub * 3 * aph + c;
    for (int s = 0; s < a.nseg; ++s) {
      a.aux_in[(bh * a.nseg + s) * aph + c] = x;
      for (int j0 = s * per; j0 < (s + 1) * per; j0 += U) {
        float p0[U], p1[U], p2[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
          // pieces past the segment's end read as the identity map
          const bool in = j0 + j < (s + 1) * per;
          const float* p = sm + static_cast<long>(in ? j0 + j : j0) * 3 * aph;
          p0[j] = in ? p[0] : 1.f;
          p1[j] = in ? p[aph] : 0.f;
          p2[j] = in ? p[2 * aph] : 0.f;
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
          if (a.gain == GAIN_PGDN) {
            x = fmaf(p0[j], x, p1[j]);
          } else {
            x = fmaf(p0[j], x, p1[j]) / fmaf(p2[j], x, 1.f);
          }
        }
      }
    }
    if (a.aux_final) a.aux_final[item] = x;
  }
  // the per-head PGDN centre, repeated for the nseg segment heads of the view
  if (a.gain == GAIN_PGDN && item < static_cast<long>(a.H) * a.nseg)
    a.mu_seg[item] = a.g.mu_log[item / a.nseg];
}

hipError_t launch_segment_stats(const StatArgs& a, hipStream_t st) {
  if (a.T > 0) {
    const unsigned nblk = static_cast<unsigned>(static_cast<long>(a.B) * a.H * (a.T / a.lsub));
    if (a.gain == GAIN_KDN_ISO) {
      if (a.dk == 128) hipLaunchKernelGGL(segment_summary_iso_kernel<128>, dim3(nblk), dim3(256), 0, st, a);
      else hipLaunchKernelGGL(segment_summary_iso_kernel<64>, dim3(nblk), dim3(256), 0, st, a);
    } else if (a.gain == GAIN_PGDN) {
      if (a.dk == 128) hipLaunchKernelGGL((segment_summary_kernel<128, GAIN_PGDN>), dim3(nblk), dim3(128), 0, st, a);
      else hipLaunchKernelGGL((segment_summary_kernel<64, GAIN_PGDN>), dim3(nblk), dim3(64), 0, st, a);
    } else {
      if (a.dk == 128) hipLaunchKernelGGL((segment_summary_kernel<128, GAIN_KDN>), dim3(nblk), dim3(128), 0, st, a);
      else hipLaunchKernelGGL((segment_summary_kernel<64, GAIN_KDN>), dim3(nblk), dim3(64), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long items = static_cast<long>(a.B) * a.H * (a.gain == GAIN_KDN_ISO ? 1 : a.dk);
  const long cover = items > static_cast<long>(a.H) * a.nseg ? items : static_cast<long>(a.H) * a.nseg;
  hipLaunchKernelGGL(segment_chain_kernel, dim3(static_cast<unsigned>((cover + 63) / 64)), dim3(64), 0,
                     st, a);
  return hipGetLastError();
}

}  // namespace dn
