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
// (2) segment_chain_kernel: per head and channel, one wavefront scans the
//     pieces' maps 64 at a time (an inclusive scan across the lanes) and
//     applies the prefixes to the carried value: the value at each segment
//     start is written for the segment's head of the [B, H nseg] view, the
//     value after the last token as aux_final.
// A summary is the map p -> (m00 p + m01) / (m10 p + 1) as three floats
// (m00, m01, m10), its matrix normalised to a (1, 1) entry of 1; PGDN's affine
// map A -> m A + c is the case (m, c, 0).  Layout [B, H, aph, T / lsub, 3].
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
  const float inv = __builtin_amdgcn_rcpf(fmaf(u, n01, 1.f));
  m00 = n00 * inv;
  m01 = n01 * inv;
  m10 = n10 * inv;
}

// PGDN and diagonal KDN: one thread per key channel, one workgroup per piece.
// The loads of U tokens are issued before their arithmetic (the composition
// is a serial chain per channel; its inputs are not).
// CHN: per-channel decay (alpha bf16 [B, H, T, dk]), else one fp32 alpha per
// token [B, H, T].
template <int DK, int GAIN, bool CHN>
__global__ __launch_bounds__(DK) __attribute__((amdgpu_waves_per_eu(1, 4))) void segment_summary_kernel(StatArgs a) {
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
    const uint16_t* al = static_cast<const uint16_t*>(a.g.alpha) + (CHN ? t0 * DK + c : 0);
    const float* als = static_cast<const float*>(a.g.alpha) + t0;
    const uint16_t* om = static_cast<const uint16_t*>(a.g.omega) + t0 * DK + c;
    float m00 = 1.f, m01 = 0.f, m10 = 0.f;
    for (int i0 = 0; i0 < a.lsub; i0 += U) {
      float kk[U], aa[U], ww[U], rr[U];
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const long o = static_cast<long>(i0 + j) * DK;
        kk[j] = bf2f(kp[o]);
        aa[j] = CHN ? bf2f(al[o]) : als[i0 + j];
        ww[j] = bf2f(om[o]);
        rr[j] = a.g.r[t0 + i0 + j];
      }
#pragma unroll
      for (int j = 0; j < U; ++j) {
        const float u = a.g.mu_info * kk[j] * kk[j] * __builtin_amdgcn_rcpf(rr[j]);
        mobius_step(m00, m01, m10, aa[j] * aa[j], ww[j], u);
      }
    }
    s0 = m00, s1 = m01, s2 = m10;
  }
  float* out = a.summ + ((bh * DK + c) * nsub + blockIdx.x % nsub) * 3;
  out[0] = s0;
  out[1] = s1;
  out[2] = s2;
}

// Isotropic KDN: each token's map from its channel sums (a group of lanes per
// token row); the piece's maps are then composed pairwise in a tree (later
// map on the left), every product renormalised to a (1, 1) entry of 1.  lsub
// is a power of two.
template <int DK, bool CHN>
__global__ __launch_bounds__(256) void segment_summary_iso_kernel(StatArgs a) {
  __shared__ float f00[256], f01[256], f10[256];
  DN_LDS_POISON(f00, sizeof(f00));
  DN_LDS_POISON(f01, sizeof(f01));
  DN_LDS_POISON(f10, sizeof(f10));
  const int i = threadIdx.x;
  const int nsub = a.T / a.lsub;
  const long bh = blockIdx.x / nsub;
  const long t0 = bh * a.T + static_cast<long>(blockIdx.x % nsub) * a.lsub;
  // channel sums of token t: the DK / 8 lanes of a row group read its
  // 16-byte pieces of k and alpha (whole rows per load instruction) and sum
  // them across the group with lane exchanges
  constexpr int LPR = DK / 8;            // lanes per row
  constexpr int RPI = 256 / LPR;         // rows per iteration of the block
  const int piece = i % LPR;
  for (int t = i / LPR; t < a.lsub; t += RPI) {
    const uint4 kv = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.k) + (t0 + t) * DK)[piece];
    const uint4 av = CHN ? reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.g.alpha) + (t0 + t) * DK)[piece]
                         : uint4{0u, 0u, 0u, 0u};
    const uint32_t kw[4] = {kv.x, kv.y, kv.z, kv.w}, aw[4] = {av.x, av.y, av.z, av.w};
    float nk = 0.f, sa = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float k0 = __uint_as_float(kw[e] << 16), k1 = __uint_as_float(kw[e] & 0xffff0000u);
      const float a0 = __uint_as_float(aw[e] << 16), a1 = __uint_as_float(aw[e] & 0xffff0000u);
      nk = fmaf(k0, k0, fmaf(k1, k1, nk));
      sa = fmaf(a0, a0, fmaf(a1, a1, sa));
    }
#pragma unroll
    for (int m = 1; m < LPR; m *= 2) {
      nk += __shfl_xor(nk, m);
      sa += __shfl_xor(sa, m);
    }
    if (piece == 0) {
      const float r = a.g.r[t0 + t];
      // scalar decay: the mean of alpha^2 over the channels is alpha^2
      const float al = CHN ? 0.f : static_cast<const float*>(a.g.alpha)[t0 + t];
      const float am = CHN ? sa * (1.f / DK) : al * al, om = static_cast<const float*>(a.g.omega)[t0 + t];
      const float u = a.g.mu_info * nk / (DK * r);
      // the token's map [[am, om], [u am, 1 + u om]] / (1 + u om)
      const float inv = 1.f / fmaf(u, om, 1.f);
      f00[t] = am * inv;
      f01[t] = om * inv;
      f10[t] = u * am * inv;
    }
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

// The composition L R of two normalised maps (L after R), renormalised.
__device__ __forceinline__ void mobius_compose(float& l00, float& l01, float& l10, float r00, float r01,
                                               float r10) {
  const float inv = 1.f / fmaf(l10, r01, 1.f);
  const float n00 = fmaf(l00, r00, l01 * r10);
  const float n01 = fmaf(l00, r01, l01);
  const float n10 = fmaf(l10, r00, r10);
  l00 = n00 * inv;
  l01 = n01 * inv;
  l10 = n10 * inv;
}

// One wavefront per (head, channel).  Round by round, lane l takes piece
// j0 + l (the identity past the last piece), the lanes' maps are scanned so
// that lane l holds pieces j0 .. j0 + l composed, and every lane applies its
// prefix to the value carried into the round.  The next round's summaries are
// loaded before the current round's scan.
__global__ __launch_bounds__(64) void segment_chain_kernel(StatArgs a) {
  const int aph = a.gain == GAIN_KDN_ISO ? 1 : a.dk;
  const int lane = threadIdx.x;
  const long item = blockIdx.x;  // head bh, channel c: item = bh aph + c
  // the per-head PGDN centre, repeated for the nseg segment heads of the view
  if (a.gain == GAIN_PGDN && item == 0)
    for (int e = lane; e < a.H * a.nseg; e += 64) a.mu_seg[e] = a.g.mu_log[e / a.nseg];
  if (item >= static_cast<long>(a.B) * a.H * aph) return;
  const long bh = item / aph;
  const int c = static_cast<int>(item % aph);
  const int nsub = a.T / a.lsub, per = nsub > 0 ? nsub / a.nseg : 1;
  float x = a.aux0 ? a.aux0[item] : 1.f;
  if (nsub == 0) {  // T = 0: every segment is empty
    for (int s = lane; s < a.nseg; s += 64) a.aux_in[(bh * a.nseg + s) * aph + c] = x;
    if (lane == 0 && a.aux_final) a.aux_final[item] = x;
    return;
  }
  if (lane == 0) a.aux_in[bh * a.nseg * aph + c] = x;
  const float* sm = a.summ + item * nsub * 3;
  float n0, n1, n2;
  auto load = [&](int j) {
    const float* p = sm + static_cast<long>(j < nsub ? j : nsub - 1) * 3;
    const float q0 = p[0], q1 = p[1], q2 = p[2];
    n0 = j < nsub ? q0 : 1.f;
    n1 = j < nsub ? q1 : 0.f;
    n2 = j < nsub ? q2 : 0.f;
  };
  load(lane);
  for (int j0 = 0; j0 < nsub; j0 += 64) {
    float m00 = n0, m01 = n1, m10 = n2;
    load(j0 + 64 + lane);
    for (int d = 1; d < 64; d *= 2) {
      const float e00 = __shfl_up(m00, d), e01 = __shfl_up(m01, d), e10 = __shfl_up(m10, d);
      if (lane >= d) mobius_compose(m00, m01, m10, e00, e01, e10);
    }
    const float y = fmaf(m00, x, m01) / fmaf(m10, x, 1.f);
    const int j = j0 + lane;
    // the value after the last piece of segment s - 1 enters segment s
    if (j < nsub && (j + 1) % per == 0 && (j + 1) / per < a.nseg)
      a.aux_in[(bh * a.nseg + (j + 1) / per) * aph + c] = y;
    x = __shfl(y, 63);
  }
  if (lane == 0 && a.aux_final) a.aux_final[item] = x;
}

hipError_t launch_segment_stats(const StatArgs& a, hipStream_t st) {
  if (a.T > 0) {
    const unsigned nblk = static_cast<unsigned>(static_cast<long>(a.B) * a.H * (a.T / a.lsub));
#define DN_SUMMARY(DKV, CH)                                                                              \
  if (a.gain == GAIN_KDN_ISO)                                                                            \
    hipLaunchKernelGGL((segment_summary_iso_kernel<DKV, CH>), dim3(nblk), dim3(256), 0, st, a);         \
  else if (a.gain == GAIN_PGDN)                                                                          \
    hipLaunchKernelGGL((segment_summary_kernel<DKV, GAIN_PGDN, CH>), dim3(nblk), dim3(DKV), 0, st, a); \
  else                                                                                                   \
    hipLaunchKernelGGL((segment_summary_kernel<DKV, GAIN_KDN, CH>), dim3(nblk), dim3(DKV), 0, st, a);
    if (a.dk == 128) {
      if (a.channel) { DN_SUMMARY(128, true) } else { DN_SUMMARY(128, false) }
    } else {
      if (a.channel) { DN_SUMMARY(64, true) } else { DN_SUMMARY(64, false) }
    }
#undef DN_SUMMARY
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long items = static_cast<long>(a.B) * a.H * (a.gain == GAIN_KDN_ISO ? 1 : a.dk);
  hipLaunchKernelGGL(segment_chain_kernel, dim3(static_cast<unsigned>(items)), dim3(64), 0, st, a);
  return hipGetLastError();
}

}  // namespace dn
