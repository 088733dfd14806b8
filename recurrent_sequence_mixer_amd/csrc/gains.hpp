// Per-element write-gain arithmetic shared by the decode, gain-prep and
// chunked-forward kernels, so all three evaluate the gains identically.
#pragma once

#include "common.hpp"

namespace dn {

enum Gain { GAIN_KLA = 0, GAIN_GDN = 1, GAIN_PGDN = 2, GAIN_KDN = 3, GAIN_EXPLICIT = 4, GAIN_KDN_ISO = 5 };
// Internal codes (not ABI values): the chunk kernel's per-channel-decay mode
// for the gains without a statistic (KLA, GDN - KDA -, explicit w): the gain
// code + GAIN_CD.
constexpr int GAIN_CD = 16;
enum GainCd { GAIN_KLA_CD = GAIN_KLA + GAIN_CD, GAIN_GDN_CD = GAIN_GDN + GAIN_CD,
              GAIN_EXPLICIT_CD = GAIN_EXPLICIT + GAIN_CD };

// KLA step size eta / (||k||^2 + eps)  (Kaczmarz Linear Attention §2.1).
__device__ __forceinline__ float kla_beta(float eta, float knorm2, float eps) {
  return eta / (knorm2 + eps);
}

// PGDN statistic update A_t = alphaP A_{t-1} + betaP k^2 and the bounded
// write scale B = exp(-log(x) * softsign(log A_t - mu))  (Preconditioned
// DeltaNet §2.4, Eq. 9).  log2x = log2(x), so exp(-ln x * s) = 2^(-log2x * s).
__device__ __forceinline__ float pgdn_stat(float A, float aP, float bP, float k) {
  return fmaf(aP, A, bP * k * k);
}
__device__ __forceinline__ float pgdn_scale(float A, float mu, float log2x) {
  const float r = logf(A) - mu;
  const float s = r / (1.0f + fabsf(r));
  return exp2f(-log2x * s);
}

// Diagonal KDN predicted variance p_hat = alpha^2 p + omega and the
// reverse-KL update with information scaling p = p_hat / (1 + u p_hat),
// u = (mu / r) k^2  (Kalman Delta Networks §2.4 Eqs. 23-30, §2.5).
__device__ __forceinline__ float kdn_predict(float a, float p, float om) {
  return fmaf(a * a, p, om);
}
// The division is the hardware reciprocal (v_rcp_f32, within 1 ulp): the
// update is contractive, so the rounding does not accumulate along the scan.
__device__ __forceinline__ float kdn_update(float p_hat, float k, float mu_over_r) {
  const float u = mu_over_r * k * k;
  return p_hat * __builtin_amdgcn_rcpf(fmaf(u, p_hat, 1.0f));
}

// Isotropic KDN, one variance b per head (Kalman Delta Networks §2.7,
// Eq. 40): predicted b_hat = mean(alpha^2) b + omega (the trace projection of
// D (b I) D + omega I), gain beta = b_hat / (r + b_hat n) with n = ||k||^2,
// and the reverse-KL update b = b_hat / (1 + u b_hat), u = mu n / (d_k r).
__device__ __forceinline__ float kdn_iso_predict(float alpha2_mean, float b, float om) {
  return fmaf(alpha2_mean, b, om);
}
__device__ __forceinline__ float kdn_iso_beta(float b_hat, float r, float n) {
  return b_hat / fmaf(b_hat, n, r);
}
__device__ __forceinline__ float kdn_iso_update(float b_hat, float n, float mu_over_dk_r) {
  return b_hat / fmaf(mu_over_dk_r * n, b_hat, 1.0f);
}

}  // namespace dn
