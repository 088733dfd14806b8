// Batched tokenwise decode step: one token for each of N sequences x H heads
// (the tokenwise step of Kaczmarz Linear Attention Algorithm 1; the same
// step with the PGDN, diagonal-KDN and isotropic-KDN gains of Preconditioned
// DeltaNet §2.4 and Kalman Delta Networks §2.4-2.5, §2.7).
//
// One workgroup per (sequence, head).  The d_k x d_v fp32 state is read from
// HBM once into registers, both readouts S^T (alpha k) and S^T (alpha q) are
// formed from that single read, and the updated state is written once:
//
//   y_k = S_dec^T k,  y_q = S_dec^T q,  e = v - y_k,
//   o   = S_t^T q = y_q + (w . q) e,    S_t = S_dec + w e^T,
//
// with S_dec = D_t S.  The kernel moves 2 d_k d_v * 4 bytes of state per
// head-step plus the token's inputs; it is bound by HBM bandwidth.
#include "common.hpp"
#include "gains.hpp"
#include "launch.hpp"

namespace dn {

template <typename IO> struct IoLoad;
template <> struct IoLoad<uint16_t> {
  static __device__ __forceinline__ float at(const void* p, long i) {
    return bf2f(static_cast<const uint16_t*>(p)[i]);
  }
  static __device__ __forceinline__ void store(void* p, long i, float x) {
    static_cast<uint16_t*>(p)[i] = f2bf(x);
  }
};
template <> struct IoLoad<float> {
  static __device__ __forceinline__ float at(const void* p, long i) {
    return static_cast<const float*>(p)[i];
  }
  static __device__ __forceinline__ void store(void* p, long i, float x) {
    static_cast<float*>(p)[i] = x;
  }
};

constexpr int DECODE_THREADS = 256;

// DV is the width of the value slice one pass of the workgroup handles (64
// or 128 columns).  WIDE: a head of d_v = a.dv columns (v_expand d_k, a
// multiple of DV) is walked slice by slice by the same workgroup, whose
// write gain is formed once; one workgroup per head keeps the in-place update
// of the gain's statistic (aux) free of races between value slices.  PAD: a
// head narrower than the instance (d_k = a.dk <= DK, d_v = a.dv <= DV, both
// multiples of 8): the missing key channels and value columns are neither
// read nor written and count as zero.  Otherwise d_k = DK, d_v = DV and
// every stride is a compile-time constant.
template <typename IO, int DK, int DV, int GAIN, bool CHANNEL, bool WIDE, bool PAD>
__global__ __launch_bounds__(DECODE_THREADS) void decode_step_kernel(DecodeArgs a) {
  constexpr int CG = DV / 4;                   // float4 column groups
  constexpr int RG = DECODE_THREADS / CG;      // row groups
  constexpr int RPT = DK / RG;                 // rows per thread
  static_assert(RPT * RG == DK, "row split");
  using L = IoLoad<IO>;

  __shared__ __align__(16) float s_a[DK], s_ak[DK], s_aq[DK], s_w[DK];
  __shared__ __align__(16) float s_v[DV], s_e[DV];
  __shared__ float s_red[DECODE_THREADS / 64][3];
  __shared__ __align__(16) f32x4 s_yk[RG][CG], s_yq[RG][CG];
  DN_LDS_POISON(s_a, sizeof(s_a));
  DN_LDS_POISON(s_ak, sizeof(s_ak));
  DN_LDS_POISON(s_aq, sizeof(s_aq));
  DN_LDS_POISON(s_w, sizeof(s_w));
  DN_LDS_POISON(s_v, sizeof(s_v));
  DN_LDS_POISON(s_e, sizeof(s_e));
  DN_LDS_POISON(s_red, sizeof(s_red));
  DN_LDS_POISON(s_yk, sizeof(s_yk));
  DN_LDS_POISON(s_yq, sizeof(s_yq));

  const int tid = threadIdx.x;
  const long nh = blockIdx.x;  // n * H + h
  const int h = static_cast<int>(nh % a.H);
  const int cg = tid % CG, rg = tid / CG;
  const int dk = PAD ? a.dk : DK;
  const int dv = WIDE || PAD ? a.dv : DV, ncg = dv / 4, nsl = PAD ? 1 : dv / DV;
  f32x4* Sp = reinterpret_cast<f32x4*>(a.S + nh * dk * dv);
  // PAD: this thread's state columns, and whether state row r exists
  const bool col_in = !PAD || cg < ncg;
  auto row_in = [&](int r) { return !PAD || (r < dk && col_in); };

  // 1. issue the state loads of the first slice first: they are the bulk of
  // the traffic.
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = row_in(rg + RG * i) ? __builtin_nontemporal_load(Sp + (rg + RG * i) * ncg + cg) : zero4();

  // 2. token inputs and the write gain (threads d < d_k own key channel d).
  float red1 = 0.f, red2 = 0.f, red3 = 0.f;
  float kd = 0.f, qd = 0.f, ad = 0.f, pre = 0.f, aux_new = 0.f, mu_over_r = 0.f;
  if (tid < DV) s_v[tid] = !PAD || tid < dv ? L::at(a.v, nh * dv + tid) : 0.f;
  if (tid < dk) {
    kd = L::at(a.k, nh * dk + tid);
    qd = L::at(a.q, nh * dk + tid);
    ad = CHANNEL ? L::at(a.alpha, nh * dk + tid) : static_cast<const float*>(a.alpha)[nh];
    if (GAIN == GAIN_KLA) {
      red1 = kd * kd;
      red2 = kd * qd;
    } else if (GAIN == GAIN_GDN) {
      red2 = kd * qd;
    } else if (GAIN == GAIN_PGDN) {
      const float A = pgdn_stat(a.aux[nh * dk + tid], a.alphaP[nh], a.betaP[nh], kd);
      aux_new = A;
      pre = a.eta[nh] * pgdn_scale(A, a.mu_log[h], a.log2x) * kd;
      red2 = pre * qd;
    } else if (GAIN == GAIN_KDN) {
      const float ph = kdn_predict(ad, a.aux[nh * dk + tid], L::at(a.omega, nh * dk + tid));
      pre = ph * kd;
      red1 = pre * kd;
      red2 = pre * qd;
      mu_over_r = a.mu_info / a.r[nh];
      aux_new = kdn_update(ph, kd, mu_over_r);
    } else if (GAIN == GAIN_KDN_ISO) {
      red1 = kd * kd;
      red2 = kd * qd;
      red3 = ad * ad;
    } else {  // explicit
      pre = L::at(a.w, nh * dk + tid);
      red2 = pre * qd;
    }
  }
  red1 = wave_sum(red1);
  red2 = wave_sum(red2);
  if (GAIN == GAIN_KDN_ISO && CHANNEL) red3 = wave_sum(red3);
  if ((tid & 63) == 0) {
    s_red[tid >> 6][0] = red1;
    s_red[tid >> 6][1] = red2;
    s_red[tid >> 6][2] = red3;
  }
  __syncthreads();
  float sum1 = 0.f, sum2 = 0.f, sum3 = 0.f;
#pragma unroll
  for (int i = 0; i < DECODE_THREADS / 64; ++i) {
    sum1 += s_red[i][0];
    sum2 += s_red[i][1];
    sum3 += s_red[i][2];
  }
  // isotropic KDN: the head's predicted variance and step size (every thread)
  float iso_beta = 0.f, iso_b = 0.f;
  if (GAIN == GAIN_KDN_ISO) {
    const float as = CHANNEL ? 0.f : static_cast<const float*>(a.alpha)[nh];
    const float a2 = CHANNEL ? sum3 / static_cast<float>(dk) : as * as;
    const float bh = kdn_iso_predict(a2, a.aux[nh], static_cast<const float*>(a.omega)[nh]);
    iso_beta = kdn_iso_beta(bh, a.r[nh], sum1);
    iso_b = kdn_iso_update(bh, sum1, a.mu_info / (dk * a.r[nh]));
  }
  float wq;  // w . q
  if (tid < dk) {
    float wd;
    if (GAIN == GAIN_KLA) {
      const float beta = kla_beta(a.eta[nh], sum1, a.eps);
      wd = beta * kd;
    } else if (GAIN == GAIN_GDN) {
      wd = a.eta[nh] * kd;
    } else if (GAIN == GAIN_KDN) {
      wd = pre / (a.r[nh] + sum1);
    } else if (GAIN == GAIN_KDN_ISO) {
      wd = iso_beta * kd;
    } else {
      wd = pre;
    }
    s_w[tid] = wd;
    s_a[tid] = ad;
    s_ak[tid] = ad * kd;
    s_aq[tid] = ad * qd;
    if (GAIN == GAIN_PGDN || GAIN == GAIN_KDN) a.aux[nh * dk + tid] = aux_new;
  } else if (PAD && tid < DK) {
    // missing key channels: no write, no decay term, no readout
    s_w[tid] = 0.f;
    s_a[tid] = 0.f;
    s_ak[tid] = 0.f;
    s_aq[tid] = 0.f;
  }
  if (GAIN == GAIN_KLA) wq = kla_beta(a.eta[nh], sum1, a.eps) * sum2;
  else if (GAIN == GAIN_GDN) wq = a.eta[nh] * sum2;
  else if (GAIN == GAIN_KDN) wq = sum2 / (a.r[nh] + sum1);
  else if (GAIN == GAIN_KDN_ISO) wq = iso_beta * sum2;
  else wq = sum2;
  const float a_scalar = CHANNEL ? 0.f : static_cast<const float*>(a.alpha)[nh];

  for (int sl = 0; sl < nsl; ++sl) {
    const int c0 = sl * DV;  // first value column of the slice
    if (sl > 0) {
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        s[i] = __builtin_nontemporal_load(Sp + (rg + RG * i) * ncg + c0 / 4 + cg);
      if (tid < DV) s_v[tid] = L::at(a.v, nh * dv + c0 + tid);
    }
    __syncthreads();  // gains, slice inputs visible; the previous slice's LDS reads done
    // isotropic KDN: every thread read the head's variance before the barrier
    // above, so it can be replaced now
    if (GAIN == GAIN_KDN_ISO && tid == 0 && sl == 0) a.aux[nh] = iso_b;

    // 3. partial readouts of the decayed state over this thread's rows.
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
    __syncthreads();

    // 4. residual and output (threads c < DV own value column c0 + c).
    if (tid < DV) {
      const int g = tid / 4, j = tid % 4;
      float yk = 0.f, yq = 0.f;
#pragma unroll
      for (int i = 0; i < RG; ++i) {
        yk += reinterpret_cast<const float*>(&s_yk[i][g])[j];
        yq += reinterpret_cast<const float*>(&s_yq[i][g])[j];
      }
      const float e = s_v[tid] - yk;
      s_e[tid] = e;
      if (!PAD || tid < dv) L::store(a.o, nh * dv + c0 + tid, fmaf(wq, e, yq));
    }
    __syncthreads();

    // 5. rank-1 write of the decayed state, one HBM write.
    const f32x4 e4 = reinterpret_cast<const f32x4*>(s_e)[cg];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + RG * i;
      const float dec = CHANNEL ? s_a[r] : a_scalar;
      const float wr = s_w[r];
      f32x4 o4;
#pragma unroll
      for (int j = 0; j < 4; ++j) o4[j] = fmaf(dec, s[i][j], wr * e4[j]);
      if (row_in(r)) __builtin_nontemporal_store(o4, Sp + r * ncg + c0 / 4 + cg);
    }
  }
}

template <typename IO, int DK, int DV, bool WIDE, bool PAD = false>
static hipError_t launch_decode_w(const DecodeArgs& a, int gain, bool channel, hipStream_t st) {
  dim3 grid(static_cast<unsigned>(a.N * a.H)), block(DECODE_THREADS);
#define DN_DEC(G, CH) \
  hipLaunchKernelGGL((decode_step_kernel<IO, DK, DV, G, CH, WIDE, PAD>), grid, block, 0, st, a)
  switch (gain) {
    case GAIN_KLA: if (channel) DN_DEC(GAIN_KLA, true); else DN_DEC(GAIN_KLA, false); break;
    case GAIN_GDN: if (channel) DN_DEC(GAIN_GDN, true); else DN_DEC(GAIN_GDN, false); break;
    case GAIN_PGDN: if (channel) DN_DEC(GAIN_PGDN, true); else DN_DEC(GAIN_PGDN, false); break;
    case GAIN_KDN: if (channel) DN_DEC(GAIN_KDN, true); else DN_DEC(GAIN_KDN, false); break;
    case GAIN_KDN_ISO: if (channel) DN_DEC(GAIN_KDN_ISO, true); else DN_DEC(GAIN_KDN_ISO, false); break;
    default: if (channel) DN_DEC(GAIN_EXPLICIT, true); else DN_DEC(GAIN_EXPLICIT, false); break;
  }
#undef DN_DEC
  return hipGetLastError();
}

template <typename IO, int DK, int DV>
static hipError_t launch_decode_io(const DecodeArgs& a, int gain, bool channel, hipStream_t st) {
  return a.dv == DV ? launch_decode_w<IO, DK, DV, false>(a, gain, channel, st)
                    : launch_decode_w<IO, DK, DV, true>(a, gain, channel, st);
}

// heads narrower than the instances (d_k, d_v multiples of 8 up to 128, not
// 64 / 128-wide): the instance of the next widths, with masking
template <typename IO>
static hipError_t launch_decode_pad(const DecodeArgs& a, int gain, bool channel, hipStream_t st) {
  if (a.dk <= 64 && a.dv <= 64) return launch_decode_w<IO, 64, 64, false, true>(a, gain, channel, st);
  if (a.dk <= 64) return launch_decode_w<IO, 64, 128, false, true>(a, gain, channel, st);
  if (a.dv <= 64) return launch_decode_w<IO, 128, 64, false, true>(a, gain, channel, st);
  return launch_decode_w<IO, 128, 128, false, true>(a, gain, channel, st);
}

hipError_t launch_decode(const DecodeArgs& a, int io_bf16, int gain, bool channel, hipStream_t st) {
  if (a.N * a.H == 0) return hipSuccess;
  if (!((a.dk == 64 || a.dk == 128) && a.dv % 64 == 0)) {
    if (a.dk > 128 || a.dv > 128 || a.dk % 8 != 0 || a.dv % 8 != 0) return hipErrorInvalidValue;
    return io_bf16 ? launch_decode_pad<uint16_t>(a, gain, channel, st)
                   : launch_decode_pad<float>(a, gain, channel, st);
  }
  // value slices of 128 columns where d_v allows, else of 64
  const bool w128 = a.dv % 128 == 0;
#define DN_SHAPE(IO)                                                                  \
  if (a.dk == 128 && w128) return launch_decode_io<IO, 128, 128>(a, gain, channel, st); \
  if (a.dk == 128) return launch_decode_io<IO, 128, 64>(a, gain, channel, st);          \
  if (a.dk == 64 && w128) return launch_decode_io<IO, 64, 128>(a, gain, channel, st);   \
  if (a.dk == 64) return launch_decode_io<IO, 64, 64>(a, gain, channel, st);
  if (io_bf16) {
    DN_SHAPE(uint16_t)
  } else {
    DN_SHAPE(float)
  }
#undef DN_SHAPE
  return hipErrorInvalidValue;
}

}  // namespace dn
