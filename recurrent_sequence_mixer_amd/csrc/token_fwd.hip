// Tokenwise forward over whole sequences for the heads the chunked kernels
// cannot evaluate: per-channel decay so strong that, referred to a point
// inside a chunk, its factors leave fp32 range (each half chunk decaying a
// channel by less than 2^-96).  The chunked kernels flag such a head, leave
// its state and statistic unwritten and its outputs NaN; this kernel then
// recomputes that head with the token recurrence itself (Kaczmarz Linear
// Attention Algorithm 1; the gains of Preconditioned DeltaNet §2.4 and Kalman
// Delta Networks §2.4-2.5, §2.7), in which every factor is a single token's
// decay and nothing overflows:
//
//   y_k = S_dec^T k,  y_q = S_dec^T q,  e = v - y_k,
//   o_t = y_q + (w . q) e,  S_t = S_dec + w e^T,  S_dec = diag(alpha_t) S.
//
// One workgroup per (batch, head, 64-column value slice) keeps its d_k x 64
// slice of S in registers for the whole sequence; a head that is not flagged
// returns at once, so the launch costs a few microseconds when no head needs
// it.  Without flags every head runs: the chunked forward's path for fp32
// io at d_k = 128, which no chunk kernel is built for (its fp32 operand tiles
// would exceed the LDS).  The gain (and its statistic) is formed per token by every slice of the
// head, identically; slice 0 writes the final statistic.  Per token: one
// reduction over the key channels, then the two readouts over the state rows,
// then the residual, the output and the rank-1 update (four barriers); the
// inputs of token t + 1 are loaded while token t is computed.
#include "common.hpp"
#include "gains.hpp"
#include "launch.hpp"

namespace dn {

namespace {

constexpr int TW_THREADS = 256;
constexpr int TW_BV = 64;  // value columns per workgroup

template <typename IO> __device__ __forceinline__ float ld(const void* p, long i);
template <> __device__ __forceinline__ float ld<uint16_t>(const void* p, long i) {
  return bf2f(static_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float ld<float>(const void* p, long i) {
  return static_cast<const float*>(p)[i];
}
template <typename IO> __device__ __forceinline__ void st(void* p, long i, float x);
template <> __device__ __forceinline__ void st<uint16_t>(void* p, long i, float x) {
  static_cast<uint16_t*>(p)[i] = f2bf(x);
}
template <> __device__ __forceinline__ void st<float>(void* p, long i, float x) {
  static_cast<float*>(p)[i] = x;
}

// the inputs of one token that a thread needs: key-channel values (threads
// d < d_k), a value column (threads c < 64) and the per-token scalars
struct TokIn {
  float k, q, a, om, w;  // channel tid: key, query, decay, KDN omega, explicit w
  float v;               // value column c0 + tid
  float eta, r, aP, bP, oms;  // scalars: eta, r, alphaP, betaP, isotropic omega
};

}  // namespace

// CHAN: per-channel decay, alpha io [B, H, T, dk]; else alpha fp32 [B, H, T]
template <typename IO, int DK, int GAIN, bool CHAN>
__global__ __launch_bounds__(TW_THREADS) void token_fwd_kernel(TokenArgs a) {
  constexpr int CG = TW_BV / 4;           // float4 column groups
  constexpr int RG = TW_THREADS / CG;     // row groups
  constexpr int RPT = DK / RG;            // state rows per thread
  static_assert(RPT * RG == DK, "row split");
  constexpr int NW = TW_THREADS / 64;

  __shared__ __align__(16) float s_a[DK], s_ak[DK], s_aq[DK], s_w[DK];
  __shared__ __align__(16) float s_e[TW_BV];
  __shared__ float s_red[NW][3];
  __shared__ __align__(16) f32x4 s_yk[RG][CG], s_yq[RG][CG];
  DN_LDS_POISON(s_a, sizeof(s_a));
  DN_LDS_POISON(s_ak, sizeof(s_ak));
  DN_LDS_POISON(s_aq, sizeof(s_aq));
  DN_LDS_POISON(s_w, sizeof(s_w));
  DN_LDS_POISON(s_e, sizeof(s_e));
  DN_LDS_POISON(s_red, sizeof(s_red));
  DN_LDS_POISON(s_yk, sizeof(s_yk));
  DN_LDS_POISON(s_yq, sizeof(s_yq));

  const int nsl = a.dv / TW_BV;
  const long bh = blockIdx.x / nsl;
  const int sl = static_cast<int>(blockIdx.x % nsl);
  const int c0 = sl * TW_BV;
  if (a.flags) {
    int any = 0;
    for (int i = 0; i < a.nflag; ++i) any |= a.flags[bh * a.nflag + i];
    if (!any) return;  // uniform over the workgroup
  }
  const int tid = threadIdx.x;
  const int h = static_cast<int>(bh % a.H);
  const int cg = tid % CG, rg = tid / CG;
  const int dv = a.dv;
  const long T = a.T;

  // the state slice: rows rg + RG i, columns c0 + 4 cg .. +3
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = a.S0 ? *reinterpret_cast<const f32x4*>(a.S0 + (bh * DK + rg + RG * i) * dv + c0 + 4 * cg)
                : zero4();
  // the statistic: per key channel (PGDN A, KDN p; thread d) or per head
  // (isotropic KDN b; every thread)
  float stat = 1.f;
  if constexpr (GAIN == GAIN_PGDN || GAIN == GAIN_KDN) {
    if (tid < DK && a.aux0) stat = a.aux0[bh * a.aux_seg * DK + tid];
  } else if constexpr (GAIN == GAIN_KDN_ISO) {
    if (a.aux0) stat = a.aux0[bh * a.aux_seg];
  }

  const long tok0 = bh * T;
  auto load = [&](long t) __attribute__((always_inline)) {
    TokIn x{};
    const long tt = tok0 + t;
    if (tid < DK) {
      x.k = ld<IO>(a.k, tt * DK + tid);
      x.q = ld<IO>(a.q, tt * DK + tid);
      x.a = CHAN ? ld<IO>(a.g.alpha, tt * DK + tid) : static_cast<const float*>(a.g.alpha)[tt];
      if constexpr (GAIN == GAIN_KDN) x.om = ld<IO>(a.g.omega, tt * DK + tid);
      if constexpr (GAIN == GAIN_EXPLICIT) x.w = ld<IO>(a.g.w, tt * DK + tid);
    }
    if (tid < TW_BV) x.v = ld<IO>(a.v, tt * dv + c0 + tid);
    if constexpr (GAIN == GAIN_KLA || GAIN == GAIN_GDN || GAIN == GAIN_PGDN) x.eta = a.g.eta[tt];
    if constexpr (GAIN == GAIN_KDN || GAIN == GAIN_KDN_ISO) x.r = a.g.r[tt];
    if constexpr (GAIN == GAIN_PGDN) {
      x.aP = a.g.alphaP[tt];
      x.bP = a.g.betaP[tt];
    }
    if constexpr (GAIN == GAIN_KDN_ISO) x.oms = static_cast<const float*>(a.g.omega)[tt];
    return x;
  };

  TokIn cur{};
  if (T > 0) cur = load(0);
  for (long t = 0; t < T; ++t) {
    const TokIn nx = load(t + 1 < T ? t + 1 : t);  // the next token's inputs, in flight

    // 1. the gain's reductions over the key channels (threads d < d_k)
    float red1 = 0.f, red2 = 0.f, red3 = 0.f, pre = 0.f, stat_new = stat, mu_over_r = 0.f;
    if (tid < DK) {
      if constexpr (GAIN == GAIN_KLA) {
        red1 = cur.k * cur.k;
        red2 = cur.k * cur.q;
      } else if constexpr (GAIN == GAIN_GDN) {
        red2 = cur.k * cur.q;
      } else if constexpr (GAIN == GAIN_PGDN) {
        stat_new = pgdn_stat(stat, cur.aP, cur.bP, cur.k);
        pre = cur.eta * pgdn_scale(stat_new, a.g.mu_log[h], a.g.log2x) * cur.k;
        red2 = pre * cur.q;
      } else if constexpr (GAIN == GAIN_KDN) {
        const float ph = kdn_predict(cur.a, stat, cur.om);
        pre = ph * cur.k;
        red1 = pre * cur.k;
        red2 = pre * cur.q;
        mu_over_r = a.g.mu_info / cur.r;
        stat_new = kdn_update(ph, cur.k, mu_over_r);
      } else if constexpr (GAIN == GAIN_KDN_ISO) {
        red1 = cur.k * cur.k;
        red2 = cur.k * cur.q;
        red3 = cur.a * cur.a;
      } else {
        pre = cur.w;
        red2 = pre * cur.q;
      }
    }
    red1 = wave_sum(red1);
    red2 = wave_sum(red2);
    if constexpr (GAIN == GAIN_KDN_ISO) red3 = wave_sum(red3);
    if ((tid & 63) == 0) {
      s_red[tid >> 6][0] = red1;
      s_red[tid >> 6][1] = red2;
      s_red[tid >> 6][2] = red3;
    }
    __syncthreads();  // (1) reductions; the previous token's update is done
    float sum1 = 0.f, sum2 = 0.f, sum3 = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      sum1 += s_red[i][0];
      sum2 += s_red[i][1];
      sum3 += s_red[i][2];
    }
    float iso_beta = 0.f;
    if constexpr (GAIN == GAIN_KDN_ISO) {
      const float bhat = kdn_iso_predict(sum3 / static_cast<float>(DK), stat, cur.oms);
      iso_beta = kdn_iso_beta(bhat, cur.r, sum1);
      stat_new = kdn_iso_update(bhat, sum1, a.g.mu_info / (DK * cur.r));
    }
    if (tid < DK) {
      float wd;
      if constexpr (GAIN == GAIN_KLA) wd = kla_beta(cur.eta, sum1, a.g.eps) * cur.k;
      else if constexpr (GAIN == GAIN_GDN) wd = cur.eta * cur.k;
      else if constexpr (GAIN == GAIN_KDN) wd = pre / (cur.r + sum1);
      else if constexpr (GAIN == GAIN_KDN_ISO) wd = iso_beta * cur.k;
      else wd = pre;
      s_w[tid] = wd;
      s_a[tid] = cur.a;
      s_ak[tid] = cur.a * cur.k;
      s_aq[tid] = cur.a * cur.q;
    }
    float wq;  // w . q
    if constexpr (GAIN == GAIN_KLA) wq = kla_beta(cur.eta, sum1, a.g.eps) * sum2;
    else if constexpr (GAIN == GAIN_GDN) wq = cur.eta * sum2;
    else if constexpr (GAIN == GAIN_KDN) wq = sum2 / (cur.r + sum1);
    else if constexpr (GAIN == GAIN_KDN_ISO) wq = iso_beta * sum2;
    else wq = sum2;
    stat = stat_new;
    __syncthreads();  // (2) w, alpha k, alpha q

    // 2. partial readouts of the decayed state over this thread's rows
    f32x4 pk = zero4(), pq = zero4();
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + RG * i;
      const float ak = s_ak[r], aq = s_aq[r];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pk[j] = fmaf(ak, s[i][j], pk[j]);
        pq[j] = fmaf(aq, s[i][j], pq[j]);
      }
    }
    s_yk[rg][cg] = pk;
    s_yq[rg][cg] = pq;
    __syncthreads();  // (3) partial readouts

    // 3. residual and output (threads c < 64 own value column c0 + c)
    if (tid < TW_BV) {
      const int g = tid / 4, j = tid % 4;
      float yk = 0.f, yq = 0.f;
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        yk += reinterpret_cast<const float*>(&s_yk[i][g])[j];
        yq += reinterpret_cast<const float*>(&s_yq[i][g])[j];
      }
      const float e = cur.v - yk;
      s_e[tid] = e;
      if (a.o) st<IO>(a.o, (tok0 + t) * dv + c0 + tid, fmaf(wq, e, yq));
    }
    __syncthreads();  // (4) residual

    // 4. rank-1 update of the decayed state
    const f32x4 e4 = reinterpret_cast<const f32x4*>(s_e)[cg];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + RG * i;
      const float dec = s_a[r], wr = s_w[r];
#pragma unroll
      for (int j = 0; j < 4; ++j) s[i][j] = fmaf(dec, s[i][j], wr * e4[j]);
    }
    cur = nx;
  }

  if (a.S_final) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *reinterpret_cast<f32x4*>(a.S_final + (bh * DK + rg + RG * i) * dv + c0 + 4 * cg) = s[i];
  }
  if (sl == 0 && a.aux_final) {
    if constexpr (GAIN == GAIN_PGDN || GAIN == GAIN_KDN) {
      if (tid < DK) a.aux_final[bh * DK + tid] = stat;
    } else if constexpr (GAIN == GAIN_KDN_ISO) {
      if (tid == 0) a.aux_final[bh] = stat;
    }
  }
}

template <typename IO, int DK, bool CHAN>
static hipError_t launch_token_dk(const TokenArgs& a, int gain, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(static_cast<long>(a.B) * a.H * (a.dv / TW_BV))),
      block(TW_THREADS);
#define DN_TW(G) hipLaunchKernelGGL((token_fwd_kernel<IO, DK, G, CHAN>), grid, block, 0, st, a)
  switch (gain) {
    case GAIN_KLA: DN_TW(GAIN_KLA); break;
    case GAIN_GDN: DN_TW(GAIN_GDN); break;
    case GAIN_PGDN: DN_TW(GAIN_PGDN); break;
    case GAIN_KDN: DN_TW(GAIN_KDN); break;
    case GAIN_KDN_ISO: DN_TW(GAIN_KDN_ISO); break;
    case GAIN_EXPLICIT: DN_TW(GAIN_EXPLICIT); break;
    default: return hipErrorInvalidValue;
  }
#undef DN_TW
  return hipGetLastError();
}

template <bool CHAN>
static hipError_t launch_token_c(const TokenArgs& a, int io_bf16, int gain, hipStream_t st) {
  if (io_bf16) {
    if (a.dk == 128) return launch_token_dk<uint16_t, 128, CHAN>(a, gain, st);
    if (a.dk == 64) return launch_token_dk<uint16_t, 64, CHAN>(a, gain, st);
    return hipErrorInvalidValue;
  }
  if (a.dk == 128) return launch_token_dk<float, 128, CHAN>(a, gain, st);
  if (a.dk == 64) return launch_token_dk<float, 64, CHAN>(a, gain, st);
  return hipErrorInvalidValue;
}

hipError_t launch_token_fwd(const TokenArgs& a, int io_bf16, int gain, bool channel, hipStream_t st) {
  if (a.B * a.H <= 0) return hipSuccess;
  if (a.dv % TW_BV != 0) return hipErrorInvalidValue;
  return channel ? launch_token_c<true>(a, io_bf16, gain, st) : launch_token_c<false>(a, io_bf16, gain, st);
}

}  // namespace dn
