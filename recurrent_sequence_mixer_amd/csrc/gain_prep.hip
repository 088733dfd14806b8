// Write-gain scans on their own (dn_gain_prep): per-token write vectors w_t,
// chunk-local cumulative log-decay, and the PGDN statistic / KDN variance
// entering each chunk.  It evaluates the same per-element gain arithmetic
// (gains.hpp) as the fused chunked forward and the decode step, so its
// outputs expose, token by token, the gains those kernels apply.
//
// One workgroup per (batch, head); thread d owns key channel d and carries
// A_t (PGDN, Preconditioned DeltaNet §2.4 Eq. 9) or p_t (diagonal KDN,
// Kalman Delta Networks §2.4-2.5) through the sequence; for isotropic KDN
// (§2.7, Eq. 40) every thread carries the head's one variance b.
#include "common.hpp"
#include "gains.hpp"
#include "launch.hpp"

namespace dn {

template <typename IO> __device__ __forceinline__ float io_at(const void* p, long i);
template <> __device__ __forceinline__ float io_at<uint16_t>(const void* p, long i) {
  return bf2f(static_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float io_at<float>(const void* p, long i) {
  return static_cast<const float*>(p)[i];
}

template <typename IO, int DK, int GAIN, bool CHANNEL>
__global__ __launch_bounds__(DK) void gain_prep_kernel(GainPrepArgs a) {
  constexpr int NW = DK / 64;
  constexpr bool ISO = GAIN == GAIN_KDN_ISO;
  constexpr bool AUX = GAIN == GAIN_PGDN || GAIN == GAIN_KDN || ISO;
  __shared__ float s_part[2][2][NW];
  DN_LDS_POISON(s_part, sizeof(s_part));
  const int d = threadIdx.x, wave = d >> 6, lane = d & 63;
  const long bh = blockIdx.x;
  const int h = static_cast<int>(bh % a.H);
  const int T = a.T;
  const int C = a.C;
  float st = a.aux0 ? a.aux0[ISO ? bh : bh * DK + d] : 1.f;
  float G = 0.f;
  const float mu = GAIN == GAIN_PGDN ? a.g.mu_log[h] : 0.f;
  for (int t = 0; t < T; ++t) {
    const long ti = bh * T + t;
    if (t % C == 0) {
      G = 0.f;
      if (a.aux_chunk && AUX && (!ISO || d == 0))
        a.aux_chunk[ISO ? bh * ((T + C - 1) / C) + t / C : (bh * ((T + C - 1) / C) + t / C) * DK + d] = st;
    }
    const float kk = io_at<IO>(a.k, ti * DK + d);
    const float al = CHANNEL ? io_at<IO>(a.g.alpha, ti * DK + d)
                             : static_cast<const float*>(a.g.alpha)[ti];
    G += logf(al);
    if (a.g_out) {
      if (CHANNEL) a.g_out[ti * DK + d] = G;
      else if (d == 0) a.g_out[ti] = G;
    }
    float pre = 0.f, red = 0.f, red2 = 0.f, wv = 0.f;
    if (GAIN == GAIN_KLA) {
      red = kk * kk;
    } else if (ISO) {
      red = kk * kk;
      red2 = al * al;
    } else if (GAIN == GAIN_PGDN) {
      st = pgdn_stat(st, a.g.alphaP[ti], a.g.betaP[ti], kk);
      wv = a.g.eta[ti] * pgdn_scale(st, mu, a.g.log2x) * kk;
    } else if (GAIN == GAIN_KDN) {
      const float ph = kdn_predict(al, st, io_at<IO>(a.g.omega, ti * DK + d));
      pre = ph * kk;
      red = pre * kk;
      st = kdn_update(ph, kk, a.g.mu_info / a.g.r[ti]);
    } else if (GAIN == GAIN_GDN) {
      wv = a.g.eta[ti] * kk;
    } else {
      wv = io_at<IO>(a.g.w, ti * DK + d);
    }
    if (GAIN == GAIN_KLA || GAIN == GAIN_KDN || ISO) {
      const float s = wave_sum(red);
      const float s2 = ISO && CHANNEL ? wave_sum(red2) : 0.f;
      if (lane == 0) {
        s_part[t & 1][0][wave] = s;
        s_part[t & 1][1][wave] = s2;
      }
      __syncthreads();
      float tot = 0.f, tot2 = 0.f;
#pragma unroll
      for (int i = 0; i < NW; ++i) {
        tot += s_part[t & 1][0][i];
        tot2 += s_part[t & 1][1][i];
      }
      if constexpr (ISO) {
        const float bh_ = kdn_iso_predict(CHANNEL ? tot2 * (1.0f / DK) : al * al, st,
                                          static_cast<const float*>(a.g.omega)[ti]);
        wv = kdn_iso_beta(bh_, a.g.r[ti], tot) * kk;
        st = kdn_iso_update(bh_, tot, a.g.mu_info / (DK * a.g.r[ti]));
      } else {
        wv = GAIN == GAIN_KLA ? kla_beta(a.g.eta[ti], tot, a.g.eps) * kk : pre / (a.g.r[ti] + tot);
      }
    }
    a.w_out[ti * DK + d] = wv;
  }
  if (a.aux_final && AUX && (!ISO || d == 0)) a.aux_final[ISO ? bh : bh * DK + d] = st;
}

template <typename IO, int DK>
static hipError_t launch_gp(const GainPrepArgs& a, int gain, bool channel, hipStream_t st) {
  dim3 grid(static_cast<unsigned>(a.B * a.H)), block(DK);
#define DN_GP(G, CHN) hipLaunchKernelGGL((gain_prep_kernel<IO, DK, G, CHN>), grid, block, 0, st, a)
  switch (gain) {
    case GAIN_KLA: if (channel) DN_GP(GAIN_KLA, true); else DN_GP(GAIN_KLA, false); break;
    case GAIN_GDN: if (channel) DN_GP(GAIN_GDN, true); else DN_GP(GAIN_GDN, false); break;
    case GAIN_PGDN: if (channel) DN_GP(GAIN_PGDN, true); else DN_GP(GAIN_PGDN, false); break;
    case GAIN_KDN: if (channel) DN_GP(GAIN_KDN, true); else DN_GP(GAIN_KDN, false); break;
    case GAIN_KDN_ISO: if (channel) DN_GP(GAIN_KDN_ISO, true); else DN_GP(GAIN_KDN_ISO, false); break;
    default: if (channel) DN_GP(GAIN_EXPLICIT, true); else DN_GP(GAIN_EXPLICIT, false); break;
  }
#undef DN_GP
  return hipGetLastError();
}

hipError_t launch_gain_prep(const GainPrepArgs& a, int io_bf16, int gain, bool channel,
                            hipStream_t st) {
  if (io_bf16) return a.dk == 128 ? launch_gp<uint16_t, 128>(a, gain, channel, st)
                                  : launch_gp<uint16_t, 64>(a, gain, channel, st);
  return a.dk == 128 ? launch_gp<float, 128>(a, gain, channel, st)
                     : launch_gp<float, 64>(a, gain, channel, st);
}

}  // namespace dn
