// Chunked backward of the gated delta-rule recurrence, scalar decay.
//
// Training differentiates the same recurrence the forward evaluates
// (Preconditioned DeltaNet §2.5: the chunk form with backpropagation; the
// chunk form itself is Kaczmarz Linear Attention §2.5 Eqs. 7-9 and
// Preconditioned DeltaNet §2.6 Eq. 6).  Per chunk of n <= 64 tokens, with
// G_t the natural-log decay from the chunk start through token t, g_t =
// exp(G_t), D_ji = exp(G_j - G_i), and the write vectors w_t:
//
//   L = strict_lower(D o (K W^T)),  M = lower(D o (Q W^T)),
//   (I + L) E = R = V - diag(g) K S_in,   O = diag(g) Q S_in + M E,
//   S_out = g_n S_in + W~^T E,   W~_i = (g_n / g_i) w_i.
//
// Given dO and dS_out the chunk's gradients are
//
//   dE = M^T dO + W~ dS_out,   (I + L)^T dR = dE,   dV = dR,
//   dS_in = g_n dS_out + (diag(g) Q)^T dO - (diag(g) K)^T dR,
//   dL = -dR E^T (strict lower),   dM = dO E^T (lower),
//   dk_t = g_t (-S_in dR_t) + sum_{i<t} D_ti dL_ti w_i,
//   dq_t = g_t (S_in dO_t) + sum_{i<=t} D_ti dM_ti w_i,
//   dw_i = (g_n / g_i) dS_out E_i + sum_{j>i} D_ji dL_ji k_j + sum_{j>=i} D_ji dM_ji q_j,
//
// and the decay's: dL/dG_t collects g_t k_t . (-S_in dR_t) + g_t q_t . (S_in dO_t),
// + (L o dL) and (M o dM) row sums minus column sums, - (g_n / g_i) w_i . (dS_out E_i)
// (with the negated sum of the last term and g_n <S_in, dS_out> going to the
// chunk's last token); dL/d log(alpha_t) is the sum of dL/dG_j over j >= t
// in the chunk.
//
// chunk_bwd_state_kernel: one workgroup per (batch, head, 32 value columns).
// The value columns of dS evolve independently, so each workgroup carries its
// slice of dS; the per-token key-side gradients (dq, dk, dw, dG) are sums
// over value columns and are accumulated over the slices with fp32 atomics.
// A forward sweep first stores the state entering every chunk and the
// residuals E; the reverse sweep then walks the chunks from the last.  All
// arithmetic is fp32 (the operands k, q, w staged in the io dtype, w rounded
// to it), one product element per thread and step from LDS.
//
// gain_bwd_kernel: one workgroup per (batch, head), one thread per key
// channel, walking the tokens backwards: the write gain's derivative
// (KLA / GDN: Kaczmarz Linear Attention §2.1; PGDN: Preconditioned DeltaNet
// §2.4, Eq. 9, the statistic recomputed per chunk from its value at the chunk
// start and differentiated backwards), and the decay's gradient from dG.
#include "common.hpp"
#include "gains.hpp"
#include "launch.hpp"

namespace dn {

namespace bwd {

constexpr int CH = 64;   // chunk length
constexpr int DVS = 32;  // value columns per workgroup
constexpr int NT = 256;  // threads of the state kernel
constexpr int PS = DVS + 1;  // row pitch of [x][DVS] fp32 arrays
constexpr int PC = CH + 1;   // row pitch of [CH][CH] fp32 arrays

template <typename E, int DK>
struct Smem {
  static constexpr int PK = DK + 2;  // row pitch of the [CH][DK] operand rows
  E k[CH * PK], q[CH * PK], w[CH * PK];
  float S[DK * PS];   // forward: the running state; reverse: S_in of the chunk
  float dS[DK * PS];  // reverse: dS carried backwards
  float e[CH * PS];   // reverse: E of the chunk
  float x[CH * PS];   // forward: R, then E in place; reverse: dO
  float y[CH * PS];   // reverse: dE, then dR in place
  float lm[CH * PC];  // L, then D o dL
  float mm[CH * PC];  // M, then D o dM
  float G[CH];        // natural-log decay from the chunk start
  float gam[CH];      // exp(G)
  float sg[CH];       // this slice's part of dL/dG per token
  float red[NT];
};

template <typename E>
__device__ __forceinline__ float ld(const void* p, long i) {
  return Elem<E>::get(static_cast<const E*>(p)[i]);
}

template <typename E, int DK>
__global__ __launch_bounds__(NT) void chunk_bwd_state_kernel(BwdArgs a) {
  using Sm = Smem<E, DK>;
  constexpr int PK = Sm::PK;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int nsl = a.dv / DVS;
  const long bh = blockIdx.x / nsl;
  const int col0 = (blockIdx.x % nsl) * DVS;
  const int T = a.T, dv = a.dv;
  const int nch = (T + CH - 1) / CH;
  const long tok0 = bh * T;

  // chunk c into LDS: k, w (and q), the decay; `x_from` fills x with v
  // (forward) or dO (reverse), rows past the end zero
  auto stage = [&](int c, bool with_q, const void* xsrc) {
    const int t0 = c * CH, n = min(CH, T - t0);
    for (int idx = tid; idx < CH * DK; idx += NT) {
      const int t = idx / DK, d = idx % DK;
      const bool ok = t < n;
      const long gi = (tok0 + t0 + t) * DK + d;
      sm.k[t * PK + d] = Elem<E>::put(ok ? ld<E>(a.k, gi) : 0.f);
      sm.w[t * PK + d] = Elem<E>::put(ok ? a.w[gi] : 0.f);
      if (with_q) sm.q[t * PK + d] = Elem<E>::put(ok ? ld<E>(a.q, gi) : 0.f);
    }
    for (int idx = tid; idx < CH * DVS; idx += NT) {
      const int t = idx / DVS, cc = idx % DVS;
      sm.x[t * PS + cc] = t < n ? ld<E>(xsrc, (tok0 + t0 + t) * dv + col0 + cc) : 0.f;
    }
    if (tid < 64) {
      // inclusive prefix sum of log(alpha) over the chunk (padding: alpha = 1)
      float l = tid < n ? logf(static_cast<const float*>(a.g.alpha)[tok0 + t0 + tid]) : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(l, off);
        if (lane >= off) l += y;
      }
      sm.G[tid] = l;
      sm.gam[tid] = expf(l);
      sm.sg[tid] = 0.f;
    }
  };
  auto dotkw = [&](const E* rows, int j, int i) {  // rows_j . w_i over DK
    float s = 0.f;
#pragma unroll 8
    for (int d = 0; d < DK; ++d) s = fmaf(Elem<E>::get(rows[j * PK + d]), Elem<E>::get(sm.w[i * PK + d]), s);
    return s;
  };

  // ---------------- forward sweep: S_in of every chunk and E
  for (int idx = tid; idx < DK * DVS; idx += NT) {
    const int d = idx / DVS, cc = idx % DVS;
    sm.S[d * PS + cc] = a.S0 ? a.S0[(bh * DK + d) * dv + col0 + cc] : 0.f;
  }
  for (int c = 0; c < nch; ++c) {
    const int t0 = c * CH, n = min(CH, T - t0);
    __syncthreads();  // the previous chunk's readers of k, w, x, S are done
    stage(c, false, a.v);
    __syncthreads();
    // S_in to the checkpoint; L; R = V - g K S_in
    for (int idx = tid; idx < DK * DVS; idx += NT) {
      const int d = idx / DVS, cc = idx % DVS;
      a.S_ck[((bh * nch + c) * DK + d) * dv + col0 + cc] = sm.S[d * PS + cc];
    }
    for (int idx = tid; idx < CH * CH; idx += NT) {
      const int j = idx / CH, i = idx % CH;
      sm.lm[j * PC + i] = i < j && j < n ? expf(sm.G[j] - sm.G[i]) * dotkw(sm.k, j, i) : 0.f;
    }
    for (int idx = tid; idx < CH * DVS; idx += NT) {
      const int t = idx / DVS, cc = idx % DVS;
      float s = 0.f;
      for (int d = 0; d < DK; ++d) s = fmaf(Elem<E>::get(sm.k[t * PK + d]), sm.S[d * PS + cc], s);
      sm.x[t * PS + cc] -= sm.gam[t] * s;
    }
    __syncthreads();
    // (I + L) E = R by forward substitution, in place; 8 threads per column
    {
      const int cc = tid >> 3, part = tid & 7;
      for (int j = 1; j < n; ++j) {
        float s = 0.f;
        for (int i = part; i < j; i += 8) s = fmaf(sm.lm[j * PC + i], sm.x[i * PS + cc], s);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        if (part == 0) sm.x[j * PS + cc] -= s;
        __syncthreads();
      }
    }
    for (int idx = tid; idx < CH * DVS; idx += NT) {
      const int t = idx / DVS, cc = idx % DVS;
      if (t < n) a.E[(tok0 + t0 + t) * dv + col0 + cc] = sm.x[t * PS + cc];
    }
    // S_out = g_n S_in + sum_t (g_n / g_t) w_t E_t^T
    const float gn = sm.gam[CH - 1];
    for (int idx = tid; idx < DK * DVS; idx += NT) {
      const int d = idx / DVS, cc = idx % DVS;
      float s = 0.f;
      for (int t = 0; t < n; ++t) s = fmaf(gn / sm.gam[t] * Elem<E>::get(sm.w[t * PK + d]), sm.x[t * PS + cc], s);
      sm.S[d * PS + cc] = fmaf(gn, sm.S[d * PS + cc], s);
    }
  }

  // ---------------- reverse sweep
  __syncthreads();
  for (int idx = tid; idx < DK * DVS; idx += NT) {
    const int d = idx / DVS, cc = idx % DVS;
    sm.dS[d * PS + cc] = a.dS_T ? a.dS_T[(bh * DK + d) * dv + col0 + cc] : 0.f;
  }
  for (int c = nch - 1; c >= 0; --c) {
    const int t0 = c * CH, n = min(CH, T - t0);
    __syncthreads();
    stage(c, true, a.dO);
    for (int idx = tid; idx < DK * DVS; idx += NT) {
      const int d = idx / DVS, cc = idx % DVS;
      sm.S[d * PS + cc] = a.S_ck[((bh * nch + c) * DK + d) * dv + col0 + cc];
    }
    for (int idx = tid; idx < CH * DVS; idx += NT) {
      const int t = idx / DVS, cc = idx % DVS;
      sm.e[t * PS + cc] = t < n ? a.E[(tok0 + t0 + t) * dv + col0 + cc] : 0.f;
    }
    __syncthreads();
    const float gn = sm.gam[CH - 1];
    // L and M
    for (int idx = tid; idx < CH * CH; idx += NT) {
      const int j = idx / CH, i = idx % CH;
      const bool in = j < n;
      const float dm = expf(sm.G[j] - sm.G[i]);
      sm.lm[j * PC + i] = in && i < j ? dm * dotkw(sm.k, j, i) : 0.f;
      sm.mm[j * PC + i] = in && i <= j ? dm * dotkw(sm.q, j, i) : 0.f;
    }
    __syncthreads();
    // dE = M^T dO + W~ dS_out
    for (int idx = tid; idx < CH * DVS; idx += NT) {
      const int i = idx / DVS, cc = idx % DVS;
      float s = 0.f;
      for (int j = i; j < n; ++j) s = fmaf(sm.mm[j * PC + i], sm.x[j * PS + cc], s);
      float s2 = 0.f;
      for (int d = 0; d < DK; ++d) s2 = fmaf(Elem<E>::get(sm.w[i * PK + d]), sm.dS[d * PS + cc], s2);
      sm.y[i * PS + cc] = i < n ? fmaf(gn / sm.gam[i], s2, s) : 0.f;
    }
    // dL/dG of the chunk end: g_n <S_in, dS_out>
    {
      float s = 0.f;
      for (int idx = tid; idx < DK * DVS; idx += NT) {
        const int d = idx / DVS, cc = idx % DVS;
        s = fmaf(sm.S[d * PS + cc], sm.dS[d * PS + cc], s);
      }
      s = wave_sum(s);
      if (lane == 0) atomicAdd(&sm.sg[CH - 1], gn * s);
    }
    __syncthreads();
    // (I + L)^T dR = dE by back substitution, in place
    {
      const int cc = tid >> 3, part = tid & 7;
      for (int j = n - 2; j >= 0; --j) {
        float s = 0.f;
        for (int i = j + 1 + part; i < n; i += 8) s = fmaf(sm.lm[i * PC + j], sm.y[i * PS + cc], s);
        s += __shfl_xor(s, 1);
        s += __shfl_xor(s, 2);
        s += __shfl_xor(s, 4);
        if (part == 0) sm.y[j * PS + cc] -= s;
        __syncthreads();
      }
    }
    // dV = dR
    for (int idx = tid; idx < CH * DVS; idx += NT) {
      const int t = idx / DVS, cc = idx % DVS;
      if (t < n) a.dv_out[(tok0 + t0 + t) * dv + col0 + cc] = sm.y[t * PS + cc];
    }
    // per (token, key channel), the parts through S_in and dS_out:
    //   dk += g_t (-S_in dR_t),  dq += g_t (S_in dO_t),  dw += (g_n / g_t) dS_out E_t;
    // their decay terms go to sg
    for (int idx = tid; idx < CH * DK; idx += NT) {
      const int t = idx / DK, d = idx % DK;
      float kh = 0.f, qh = 0.f, tw = 0.f;
      for (int cc = 0; cc < DVS; ++cc) {
        const float sv = sm.S[d * PS + cc];
        kh = fmaf(-sm.y[t * PS + cc], sv, kh);
        qh = fmaf(sm.x[t * PS + cc], sv, qh);
        tw = fmaf(sm.e[t * PS + cc], sm.dS[d * PS + cc], tw);
      }
      if (t < n) {
        const long gi = (tok0 + t0 + t) * DK + d;
        const float g = sm.gam[t], f = gn / g;
        atomicAdd(&a.dk_out[gi], g * kh);
        atomicAdd(&a.dq_out[gi], g * qh);
        atomicAdd(&a.dw_acc[gi], f * tw);
        const float wtw = f * Elem<E>::get(sm.w[t * PK + d]) * tw;
        const float sgt = g * (Elem<E>::get(sm.k[t * PK + d]) * kh + Elem<E>::get(sm.q[t * PK + d]) * qh) - wtw;
        atomicAdd(&sm.sg[t], sgt);
        atomicAdd(&sm.sg[CH - 1], wtw);
      }
    }
    __syncthreads();
    // dS_in = g_n dS_out + sum_t g_t (q_t dO_t^T - k_t dR_t^T)
    for (int idx = tid; idx < DK * DVS; idx += NT) {
      const int d = idx / DVS, cc = idx % DVS;
      float s = 0.f;
      for (int t = 0; t < n; ++t)
        s = fmaf(sm.gam[t], Elem<E>::get(sm.q[t * PK + d]) * sm.x[t * PS + cc] -
                                Elem<E>::get(sm.k[t * PK + d]) * sm.y[t * PS + cc], s);
      sm.dS[d * PS + cc] = fmaf(gn, sm.dS[d * PS + cc], s);
    }
    // dL = -dR E^T, dM = dO E^T: their decay terms (L o dL, M o dM: + to the
    // row token, - to the column token), then L <- D o dL, M <- D o dM
    for (int idx = tid; idx < CH * CH; idx += NT) {
      const int j = idx / CH, i = idx % CH;
      if (j >= n || i > j) continue;
      float dl = 0.f, dmv = 0.f;
      for (int cc = 0; cc < DVS; ++cc) {
        const float ev = sm.e[i * PS + cc];
        dl = fmaf(-sm.y[j * PS + cc], ev, dl);
        dmv = fmaf(sm.x[j * PS + cc], ev, dmv);
      }
      const float dm = expf(sm.G[j] - sm.G[i]);
      const float tl = i < j ? sm.lm[j * PC + i] * dl : 0.f, tm = sm.mm[j * PC + i] * dmv;
      if (i < j) {
        atomicAdd(&sm.sg[j], tl + tm);
        atomicAdd(&sm.sg[i], -(tl + tm));
      }
      sm.lm[j * PC + i] = i < j ? dm * dl : 0.f;
      sm.mm[j * PC + i] = dm * dmv;
    }
    __syncthreads();
    // dk += sum_{i<t} (D o dL)_ti w_i,  dq += sum_{i<=t} (D o dM)_ti w_i,
    // dw_i += sum_{j>i} (D o dL)_ji k_j + sum_{j>=i} (D o dM)_ji q_j
    for (int idx = tid; idx < CH * DK; idx += NT) {
      const int t = idx / DK, d = idx % DK;
      if (t >= n) continue;
      float sk = 0.f, sq = 0.f, sw = 0.f;
      for (int i = 0; i <= t; ++i) {
        const float wv = Elem<E>::get(sm.w[i * PK + d]);
        sk = fmaf(sm.lm[t * PC + i], wv, sk);
        sq = fmaf(sm.mm[t * PC + i], wv, sq);
      }
      for (int j = t; j < n; ++j)
        sw = fmaf(sm.lm[j * PC + t], Elem<E>::get(sm.k[j * PK + d]),
                  fmaf(sm.mm[j * PC + t], Elem<E>::get(sm.q[j * PK + d]), sw));
      const long gi = (tok0 + t0 + t) * DK + d;
      atomicAdd(&a.dk_out[gi], sk);
      atomicAdd(&a.dq_out[gi], sq);
      atomicAdd(&a.dw_acc[gi], sw);
    }
    // dL/dG of the chunk to HBM; the padding tokens of a partial chunk share
    // the last real token's decay
    if (tid < CH) {
      const float v = sm.sg[tid];
      const float tail = tid == n - 1 ? [&] {
        float s = 0.f;
        for (int t = n; t < CH; ++t) s += sm.sg[t];
        return s;
      }() : 0.f;
      if (tid < n) atomicAdd(&a.dG[tok0 + t0 + tid], v + tail);
    }
  }
  __syncthreads();
  if (a.dS0)
    for (int idx = tid; idx < DK * DVS; idx += NT) {
      const int d = idx / DVS, cc = idx % DVS;
      a.dS0[(bh * DK + d) * dv + col0 + cc] = sm.dS[d * PS + cc];
    }
}

// ---------------------------------------------------------------------------
// Back through the write gains and the decay.  Thread d owns key channel d.
template <typename E, int DK, int GAIN>
__global__ __launch_bounds__(DK) void gain_bwd_kernel(GainBwdArgs a) {
  constexpr int NW = DK / 64;
  constexpr bool PG = GAIN == GAIN_PGDN;
  __shared__ float red[4][NW];
  __shared__ float As[PG ? CH : 1][PG ? DK : 1];
  const int d = threadIdx.x, wave = d >> 6, lane = d & 63;
  const long bh = blockIdx.x;
  const int h = static_cast<int>(bh % a.H);
  const int T = a.T, nch = (T + CH - 1) / CH;
  const float* alpha = static_cast<const float*>(a.g.alpha);
  // sums over the key channels of up to four values, in every thread
  auto reduce4 = [&](float& v0, float& v1, float& v2, float& v3) {
    float v[4] = {wave_sum(v0), wave_sum(v1), wave_sum(v2), wave_sum(v3)};
    __syncthreads();  // the previous round's readers are done
    if (lane == 0)
      for (int i = 0; i < 4; ++i) red[i][wave] = v[i];
    __syncthreads();
    float s[4] = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < 4; ++i)
      for (int w_ = 0; w_ < NW; ++w_) s[i] += red[i][w_];
    v0 = s[0], v1 = s[1], v2 = s[2], v3 = s[3];
  };
  float dA = PG && a.daux_T ? a.daux_T[bh * DK + d] : 0.f;  // dL/dA_t carried backwards
  float dmu = 0.f;
  const float mu = PG ? a.g.mu_log[h] : 0.f;
  const float lnx = PG ? a.g.log2x * 0.69314718055994531f : 0.f;
  for (int c = nch - 1; c >= 0; --c) {
    const int t0 = c * CH, n = min(CH, T - t0);
    if constexpr (PG) {
      // the statistic of the chunk's tokens, from its value at the chunk start
      __syncthreads();
      float A = a.aux_chunk[(bh * nch + c) * DK + d];
      for (int j = 0; j < n; ++j) {
        const long ti = bh * T + t0 + j;
        const float kk = Elem<E>::get(static_cast<const E*>(a.k)[ti * DK + d]);
        A = fmaf(a.g.alphaP[ti], A, a.g.betaP[ti] * kk * kk);
        As[j][d] = A;
      }
    }
    float sfx = 0.f;  // dL/d log(alpha) summed from the chunk end
    for (int j = n - 1; j >= 0; --j) {
      const long ti = bh * T + t0 + j;
      const float kk = Elem<E>::get(static_cast<const E*>(a.k)[ti * DK + d]);
      const float dw = a.dw_acc[ti * DK + d];
      float dkv = a.dk_out[ti * DK + d];
      sfx += a.dG[ti];
      if (d == 0) a.dalpha[ti] = sfx / alpha[ti];
      if constexpr (GAIN == GAIN_KLA) {
        // w = beta k, beta = eta / (n + eps), n = ||k||^2
        float n2 = kk * kk, db = dw * kk, z0 = 0.f, z1 = 0.f;
        reduce4(n2, db, z0, z1);
        const float et = a.g.eta[ti], den = n2 + a.g.eps;
        const float beta = et / den;
        dkv = fmaf(beta, dw, fmaf(2.f * kk, db * (-et / (den * den)), dkv));
        if (d == 0) a.deta[ti] = db / den;
      } else if constexpr (GAIN == GAIN_GDN) {
        float db = dw * kk, z0 = 0.f, z1 = 0.f, z2 = 0.f;
        reduce4(db, z0, z1, z2);
        dkv = fmaf(a.g.eta[ti], dw, dkv);
        if (d == 0) a.deta[ti] = db;
      } else if constexpr (GAIN == GAIN_EXPLICIT) {
        a.dw_out[ti * DK + d] = dw;
      } else if constexpr (PG) {
        // A_t = alphaP A_{t-1} + betaP k^2;  r = log A_t - mu;  s = r / (1 + |r|);
        // B = exp(-log(x) s);  w = eta B k
        const float A = As[j][d];
        const float Ap = j > 0 ? As[j - 1][d] : a.aux_chunk[(bh * nch + c) * DK + d];
        const float rr = logf(A) - mu;
        const float s = rr / (1.f + fabsf(rr));
        const float Bv = expf(-lnx * s);
        const float et = a.g.eta[ti], aP = a.g.alphaP[ti], bP = a.g.betaP[ti];
        float de = dw * Bv * kk;
        dkv = fmaf(et * Bv, dw, dkv);
        const float ds = et * kk * dw * Bv * (-lnx);
        const float q1 = 1.f + fabsf(rr);
        const float drr = ds / (q1 * q1);
        dmu -= drr;
        dA += drr / A;
        float daP = dA * Ap, dbP = dA * kk * kk, z0 = 0.f;
        dkv = fmaf(dA * bP, 2.f * kk, dkv);
        dA *= aP;
        reduce4(de, daP, dbP, z0);
        if (d == 0) {
          a.deta[ti] = de;
          a.dalphaP[ti] = daP;
          a.dbetaP[ti] = dbP;
        }
      }
      a.dk_out[ti * DK + d] = dkv;
    }
  }
  if constexpr (PG) {
    if (a.daux0) a.daux0[bh * DK + d] = dA;
    float z0 = 0.f, z1 = 0.f, z2 = 0.f;
    reduce4(dmu, z0, z1, z2);
    if (d == 0) atomicAdd(&a.dmu_log[h], dmu);
  }
}

__global__ void zero_kernel(float* p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0.f;
}

}  // namespace bwd

template <typename E, int DK>
static hipError_t launch_bwd_state_t(const BwdArgs& a, hipStream_t st) {
  using Sm = bwd::Smem<E, DK>;
  static_assert(sizeof(Sm) <= 160 * 1024, "LDS budget");
  auto kern = bwd::chunk_bwd_state_kernel<E, DK>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(sizeof(Sm)));
  if (err != hipSuccess) return err;
  const unsigned grid = static_cast<unsigned>(static_cast<long>(a.B) * a.H * (a.dv / bwd::DVS));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(bwd::NT), sizeof(Sm), st, a);
  return hipGetLastError();
}

hipError_t launch_chunk_bwd_state(const BwdArgs& a, int io_bf16, hipStream_t st) {
  if (a.T == 0 || a.B * a.H == 0) return hipSuccess;
  if (io_bf16) return a.dk == 128 ? launch_bwd_state_t<uint16_t, 128>(a, st) : launch_bwd_state_t<uint16_t, 64>(a, st);
  if (a.dk == 64) return launch_bwd_state_t<float, 64>(a, st);
  return hipErrorInvalidValue;
}

template <typename E, int DK>
static hipError_t launch_gain_bwd_t(const GainBwdArgs& a, int gain, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.B * a.H)), block(DK);
  switch (gain) {
    case GAIN_KLA: hipLaunchKernelGGL((bwd::gain_bwd_kernel<E, DK, GAIN_KLA>), grid, block, 0, st, a); break;
    case GAIN_GDN: hipLaunchKernelGGL((bwd::gain_bwd_kernel<E, DK, GAIN_GDN>), grid, block, 0, st, a); break;
    case GAIN_PGDN: hipLaunchKernelGGL((bwd::gain_bwd_kernel<E, DK, GAIN_PGDN>), grid, block, 0, st, a); break;
    case GAIN_EXPLICIT: hipLaunchKernelGGL((bwd::gain_bwd_kernel<E, DK, GAIN_EXPLICIT>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gain_bwd(const GainBwdArgs& a, int io_bf16, int gain, hipStream_t st) {
  if (a.T == 0 && gain != GAIN_PGDN) return hipSuccess;
  if (io_bf16) return a.dk == 128 ? launch_gain_bwd_t<uint16_t, 128>(a, gain, st) : launch_gain_bwd_t<uint16_t, 64>(a, gain, st);
  if (a.dk == 64) return launch_gain_bwd_t<float, 64>(a, gain, st);
  return hipErrorInvalidValue;
}

hipError_t launch_zero(float* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(bwd::zero_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace dn
