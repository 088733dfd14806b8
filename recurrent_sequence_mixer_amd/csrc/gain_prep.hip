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
// gain_prep_tok_kernel below.  The tokens are walked in blocks of TB: each
// block's k (and per-channel decay and KDN omega) rows and per-token gates
// are staged into LDS with 16-byte loads first, so that a block costs one
// round trip to memory rather than one per token.
template <typename IO, int DK, int GAIN, bool CHANNEL>
__global__ __launch_bounds__(DK) void gain_prep_kernel(GainPrepArgs a) {
  constexpr int NW = DK / 64;
  constexpr bool ISO = GAIN == GAIN_KDN_ISO, KD = GAIN == GAIN_KDN, PG = GAIN == GAIN_PGDN;
  constexpr bool AUX = PG || KD || ISO;
  constexpr int TB = 128 / sizeof(IO);  // tokens per staged block: 16 KiB of k rows at d_k 128
  constexpr int PV = 16 / sizeof(IO);   // elements per 16-byte piece
  constexpr int NP = TB * DK / PV / DK; // pieces per thread and array
  __shared__ float s_part[2][2][NW];
  __shared__ __align__(16) IO s_k[TB * DK];
  __shared__ __align__(16) IO s_a[CHANNEL ? TB * DK : PV];  // per-channel decay
  __shared__ __align__(16) IO s_o[KD ? TB * DK : PV];       // KDN omega
  // per token: 0 alpha (scalar decay); 1 eta (PGDN) or r (KDN modes); 2
  // alphaP (PGDN) or omega (isotropic KDN); 3 betaP (PGDN)
  __shared__ float s_g[4][TB];
  DN_LDS_POISON(s_part, sizeof(s_part));
  DN_LDS_POISON(s_k, sizeof(s_k));
  DN_LDS_POISON(s_a, sizeof(s_a));
  DN_LDS_POISON(s_o, sizeof(s_o));
  DN_LDS_POISON(s_g, sizeof(s_g));
  const int d = threadIdx.x, wave = d >> 6, lane = d & 63;
  const long bh = blockIdx.x;
  const int h = static_cast<int>(bh % a.H);
  const int T = a.T;
  const int C = a.C;
  float st = a.aux0 ? a.aux0[ISO ? bh : bh * DK + d] : 1.f;
  float G = 0.f;
  const float mu = PG ? a.g.mu_log[h] : 0.f;
  for (int tb0 = 0; tb0 < T; tb0 += TB) {
    const int nb = min(TB, T - tb0);
    const long r0 = bh * T + tb0;
    __syncthreads();  // the previous block's readers are done
    {
      // every load unconditional: rows past the block's end read its last row
      // (never used)
      auto stage = [&](const void* src, IO* dst) {
        u32x4 v[NP];
#pragma unroll
        for (int m = 0; m < NP; ++m) {
          const int i = d + DK * m, t = i / (DK / PV), c = i % (DK / PV) * PV;
          v[m] = *reinterpret_cast<const u32x4*>(static_cast<const IO*>(src) + (r0 + min(t, nb - 1)) * DK + c);
        }
#pragma unroll
        for (int m = 0; m < NP; ++m) {
          const int i = d + DK * m, t = i / (DK / PV), c = i % (DK / PV) * PV;
          *reinterpret_cast<u32x4*>(dst + t * DK + c) = v[m];
        }
      };
      stage(a.k, s_k);
      if constexpr (CHANNEL) stage(a.g.alpha, s_a);
      if constexpr (KD) stage(a.g.omega, s_o);
      for (int i = d; i < TB; i += DK) {
        const long ti = r0 + min(i, nb - 1);
        if constexpr (!CHANNEL) s_g[0][i] = static_cast<const float*>(a.g.alpha)[ti];
        if constexpr (PG) {
          s_g[1][i] = a.g.eta[ti];
          s_g[2][i] = a.g.alphaP[ti];
          s_g[3][i] = a.g.betaP[ti];
        } else {
          s_g[1][i] = a.g.r[ti];
          if constexpr (ISO) s_g[2][i] = static_cast<const float*>(a.g.omega)[ti];
        }
      }
    }
    __syncthreads();
    for (int tt = 0; tt < nb; ++tt) {
      const int t = tb0 + tt;
      const long ti = r0 + tt;
      if (t % C == 0) {
        G = 0.f;
        if (a.aux_chunk && AUX && (!ISO || d == 0))
          a.aux_chunk[ISO ? bh * ((T + C - 1) / C) + t / C : (bh * ((T + C - 1) / C) + t / C) * DK + d] = st;
      }
      const float kk = Elem<IO>::get(s_k[tt * DK + d]);
      const float al = CHANNEL ? Elem<IO>::get(s_a[tt * DK + d]) : s_g[0][tt];
      if (a.g_out) {
        G += logf(al);
        if (CHANNEL) a.g_out[ti * DK + d] = G;
        else if (d == 0) a.g_out[ti] = G;
      }
      float pre = 0.f, red = 0.f, red2 = 0.f, wv = 0.f;
      if (ISO) {
        red = kk * kk;
        red2 = al * al;
      } else if (PG) {
        st = pgdn_stat(st, s_g[2][tt], s_g[3][tt], kk);
        wv = s_g[1][tt] * pgdn_scale(st, mu, a.g.log2x) * kk;
      } else if (KD) {
        const float ph = kdn_predict(al, st, Elem<IO>::get(s_o[tt * DK + d]));
        pre = ph * kk;
        red = pre * kk;
        st = kdn_update(ph, kk, a.g.mu_info / s_g[1][tt]);
      }
      if (KD || ISO) {
        const float sm = wave_sum(red);
        const float s2 = ISO && CHANNEL ? wave_sum(red2) : 0.f;
        if (lane == 0) {
          s_part[t & 1][0][wave] = sm;
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
          const float bh_ = kdn_iso_predict(CHANNEL ? tot2 * (1.0f / DK) : al * al, st, s_g[2][tt]);
          wv = kdn_iso_beta(bh_, s_g[1][tt], tot) * kk;
          st = kdn_iso_update(bh_, tot, a.g.mu_info / (DK * s_g[1][tt]));
        } else {
          wv = pre / (s_g[1][tt] + tot);
        }
      }
      if (a.w_bf16)
        a.w_bf16[ti * DK + d] = f2bf(wv);
      else
        a.w_out[ti * DK + d] = wv;
    }
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
