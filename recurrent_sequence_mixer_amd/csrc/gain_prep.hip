// Write-gain scans on their own (dn_gain_prep): per-token write vectors w_t,
// chunk-local cumulative log-decay, and the PGDN statistic / KDN variance
// entering each chunk.  It evaluates the same per-element gain arithmetic
// (gains.hpp) as the fused chunked forward and the decode step, so its
// outputs expose, token by token, the gains those kernels apply.
//
// Gains with a statistic (gain_prep_kernel): one workgroup per (batch, head)
// - or per chunk, from the statistic entering it - whose thread d owns key
// channel d and carries A_t (PGDN, Preconditioned DeltaNet §2.4 Eq. 9) or p_t
// (diagonal KDN, Kalman Delta Networks §2.4-2.5) through the tokens; for
// isotropic KDN (§2.7, Eq. 40) every thread carries the head's one variance
// b.  KLA, GDN and explicit w (gain_prep_tok_kernel): one workgroup per chunk,
// token-parallel.
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

// The gains with a statistic (PGDN, KDN, isotropic KDN); the others take
// gain_prep_tok_kernel below.
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
    if (ISO) {
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
    }
    if (GAIN == GAIN_KDN || ISO) {
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
        wv = pre / (a.g.r[ti] + tot);
      }
    }
    if (a.w_bf16)
      a.w_bf16[ti * DK + d] = f2bf(wv);
    else
      a.w_out[ti * DK + d] = wv;
  }
  if (a.aux_final && AUX && (!ISO || d == 0)) a.aux_final[ISO ? bh : bh * DK + d] = st;
}

// N consecutive elements of an io array from element offset `off` as fp32
// (16-byte loads; off and N multiples of 8 elements)
template <typename IO, int N>
__device__ __forceinline__ void load_row(const void* base, long off, float (&v)[N]) {
  if constexpr (sizeof(IO) == 2) {
    const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int i = 0; i < N / 8; ++i) {
      const u32x4 x = p[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * i + 2 * j] = __uint_as_float(x[j] << 16);
        v[8 * i + 2 * j + 1] = __uint_as_float(x[j] & 0xFFFF0000u);
      }
    }
  } else {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off);
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const f32x4 x = p[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * i + j] = x[j];
    }
  }
}

// The gains without a statistic (KLA, GDN, explicit w) token-parallel: one
// workgroup per chunk of C tokens, four threads per token, each with a
// quarter of the key channels; ||k_t||^2 is a sum over the token's four
// lanes.  The in-chunk cumulative log-decay (g_out) is a prefix over the
// chunk's tokens: one wavefront's for scalar decay, per channel through LDS
// for per-channel decay.  Same arithmetic as gain_prep_kernel (gains.hpp),
// summed in another order.
template <typename IO, int DK, int GAIN, bool CHANNEL>
__global__ __launch_bounds__(256) void gain_prep_tok_kernel(GainPrepArgs a) {
  constexpr int DQ = DK / 4;  // key channels per thread
  __shared__ float s_g[CHANNEL ? 64 * DK : 1];
  DN_LDS_POISON(s_g, sizeof(s_g));
  const int C = a.C, T = a.T;
  const int nch = (T + C - 1) / C;
  const long bh = blockIdx.x / nch;
  const int c = static_cast<int>(blockIdx.x % nch);
  const int t0 = c * C, n = min(C, T - t0);
  const int tid = threadIdx.x, tl = tid >> 2, q = tid & 3, d0 = q * DQ;
  const bool ok = tl < n;
  const long ti = bh * T + t0 + tl;
  if (ok) {
    float kv[DQ], w[DQ];
    load_row<IO, DQ>(a.k, ti * DK + d0, kv);
    if constexpr (GAIN == GAIN_KLA) {
      float n2 = 0.f;
#pragma unroll
      for (int i = 0; i < DQ; ++i) n2 = fmaf(kv[i], kv[i], n2);
      n2 += __shfl_xor(n2, 1);
      n2 += __shfl_xor(n2, 2);
      const float beta = kla_beta(a.g.eta[ti], n2, a.g.eps);
#pragma unroll
      for (int i = 0; i < DQ; ++i) w[i] = beta * kv[i];
    } else if constexpr (GAIN == GAIN_GDN) {
      const float et = a.g.eta[ti];
#pragma unroll
      for (int i = 0; i < DQ; ++i) w[i] = et * kv[i];
    } else {
      load_row<IO, DQ>(a.g.w, ti * DK + d0, w);
    }
    if (a.w_bf16) {
      u32x4* wo = reinterpret_cast<u32x4*>(a.w_bf16 + ti * DK + d0);
#pragma unroll
      for (int i = 0; i < DQ / 8; ++i)
        wo[i] = u32x4{pack_bf2(w[8 * i], w[8 * i + 1]), pack_bf2(w[8 * i + 2], w[8 * i + 3]),
                      pack_bf2(w[8 * i + 4], w[8 * i + 5]), pack_bf2(w[8 * i + 6], w[8 * i + 7])};
    } else {
      f32x4* wo = reinterpret_cast<f32x4*>(a.w_out + ti * DK + d0);
#pragma unroll
      for (int i = 0; i < DQ / 4; ++i) wo[i] = f32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
    }
  }
  // (the four lanes of a token share `ok`, so its lane sums stay inside it)
  if (!a.g_out) return;  // uniform
  if constexpr (CHANNEL) {
    // log alpha of the thread's elements into LDS, then one thread per
    // channel runs the prefix over the chunk's tokens
    if (ok) {
      float al[DQ];
      load_row<IO, DQ>(a.g.alpha, ti * DK + d0, al);
#pragma unroll
      for (int i = 0; i < DQ; ++i) s_g[tl * DK + d0 + i] = logf(al[i]);
    }
    __syncthreads();
    if (tid < DK) {
      float G = 0.f;
      for (int t = 0; t < n; ++t) {
        G += s_g[t * DK + tid];
        a.g_out[(bh * T + t0 + t) * DK + tid] = G;
      }
    }
  } else {
    if (tid < 64) {
      // lane t: token t of the chunk (log 1 = 0 past the end)
      float G = tid < n ? logf(static_cast<const float*>(a.g.alpha)[bh * T + t0 + tid]) : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(G, off);
        if (tid >= off) G += y;
      }
      if (tid < n) a.g_out[bh * T + t0 + tid] = G;
    }
  }
}

template <typename IO, int DK>
static hipError_t launch_gp(const GainPrepArgs& a, int gain, bool channel, hipStream_t st) {
  if (gain == GAIN_KLA || gain == GAIN_GDN || gain == GAIN_EXPLICIT) {
    // token-parallel, one workgroup per chunk
    const long nch = (a.T + a.C - 1) / a.C;
    if (nch == 0) return hipSuccess;
    const dim3 grid(static_cast<unsigned>(static_cast<long>(a.B) * a.H * nch)), block(4 * a.C);
#define DN_GPT(G, CHN) hipLaunchKernelGGL((gain_prep_tok_kernel<IO, DK, G, CHN>), grid, block, 0, st, a)
    switch (gain) {
      case GAIN_KLA: if (channel) DN_GPT(GAIN_KLA, true); else DN_GPT(GAIN_KLA, false); break;
      case GAIN_GDN: if (channel) DN_GPT(GAIN_GDN, true); else DN_GPT(GAIN_GDN, false); break;
      default: if (channel) DN_GPT(GAIN_EXPLICIT, true); else DN_GPT(GAIN_EXPLICIT, false); break;
    }
#undef DN_GPT
    return hipGetLastError();
  }
  dim3 grid(static_cast<unsigned>(a.B * a.H)), block(DK);
#define DN_GP(G, CHN) hipLaunchKernelGGL((gain_prep_kernel<IO, DK, G, CHN>), grid, block, 0, st, a)
  switch (gain) {
    case GAIN_PGDN: if (channel) DN_GP(GAIN_PGDN, true); else DN_GP(GAIN_PGDN, false); break;
    case GAIN_KDN: if (channel) DN_GP(GAIN_KDN, true); else DN_GP(GAIN_KDN, false); break;
    case GAIN_KDN_ISO: if (channel) DN_GP(GAIN_KDN_ISO, true); else DN_GP(GAIN_KDN_ISO, false); break;
    default: return hipErrorInvalidValue;
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
