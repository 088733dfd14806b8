// Chunked backward of the gated delta-rule recurrence.
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
// With per-channel decay every product above carries the decay per key
// channel: g_t, D_ji and g_n / g_i become vectors over d_k applied inside the
// contractions, and dL/dG is per (token, channel).  The operands are then
// staged scaled relative to the chunk's token 31, k^ = k exp(G_t - G_r),
// q^ = q exp(G_t - G_r), w^ = w exp(G_r - G_t), so that K^ W^^T already holds
// the decay; S enters scaled by exp(G_r) and leaves by exp(G_n - G_r).  The
// L / M terms of dL/dG then reduce per element to k^ . (dL W^) + q^ . (dM W^)
// for the row token and -w^ . (dL^T K^ + dM^T Q^) for the column token.  The
// factors stay finite while each half-chunk decay of a channel is at least
// 2^-96, the range of the chunked forward; beyond it the reference is NaN.
//
// chunk_bwd_state_kernel: one workgroup per (batch, head, DVS value
// columns).  The value columns of dS evolve independently, so each
// workgroup carries its slice of dS; the per-token key-side gradients (dq,
// dk, dw, dG) are sums over value columns and are accumulated over the
// slices with fp32 atomics.  A forward sweep first stores the state entering
// every chunk and the residuals E; the reverse sweep then walks the chunks
// from the last.  All arithmetic is fp32 (the operands k, q, w staged in the
// io dtype, w rounded to it), one product element per thread and step from
// LDS.
//
// gain_bwd_kernel: one workgroup per (batch, head), one thread per key
// channel, walking the tokens backwards: the write gain's derivative
// (KLA / GDN: Kaczmarz Linear Attention §2.1; PGDN: Preconditioned DeltaNet
// §2.4, Eq. 9; KDN: Kalman Delta Networks §2.4, Eqs. 23-30 with the
// information scaling of §2.5; isotropic KDN: §2.7, Eq. 40 - the gain scan
// differentiated backwards, Appendix D), the statistic recomputed per chunk
// from its value at the chunk start, and the decay's gradient from dG.
#include "common.hpp"
#include "gains.hpp"
#include "launch.hpp"

namespace dn {

namespace bwd {

constexpr int CH = 64;      // chunk length
constexpr int NT = 256;     // threads of the state kernel
constexpr int PC = CH + 1;  // row pitch of [CH][CH] fp32 arrays
constexpr int RT = 31;      // reference token of the per-channel decay factors

template <typename E, int DK, bool CHAN>
struct Smem {
  static constexpr int DVS = CHAN ? 16 : 32;  // value columns per workgroup
  static constexpr int PS = DVS + 1;          // row pitch of [x][DVS] fp32 arrays
  static constexpr int PK = DK + 2;           // row pitch of the [CH][DK] operand rows
  static constexpr int PG = DK + 1;           // row pitch of the per-channel decay
  E k[CH * PK], q[CH * PK], w[CH * PK];  // channel decay: k^, q^, w^
  float S[DK * PS];   // forward: the running state; reverse: S_in of the chunk
  float dS[DK * PS];  // reverse: dS carried backwards
  float e[CH * PS];   // reverse: E of the chunk
  float x[CH * PS];   // forward: R, then E in place; reverse: dO
  float y[CH * PS];   // reverse: dE, then dR in place
  float lm[CH * PC];  // L, then (D o) dL
  float mm[CH * PC];  // M, then (D o) dM
  // channel decay: G per (token, channel), exp(G_r), exp(G_n - G_r), and
  // dL/dG of the chunk's last token per channel
  float Gc[CHAN ? CH * PG : 1];
  float gref[CHAN ? DK : 1], gnr[CHAN ? DK : 1], endc[CHAN ? DK : 1];
  // scalar decay: G, exp(G) and this slice's part of dL/dG per token
  float G[CH], gam[CH], sg[CH];
};

template <typename E>
__device__ __forceinline__ float ld(const void* p, long i) {
  return Elem<E>::get(static_cast<const E*>(p)[i]);
}

template <typename E, int DK, bool CHAN>
__global__ __launch_bounds__(NT) void chunk_bwd_state_kernel(BwdArgs a) {
  using Sm = Smem<E, DK, CHAN>;
  constexpr int PK = Sm::PK, PS = Sm::PS, PG = Sm::PG, DVS = Sm::DVS;
  constexpr int TPC = NT / DVS;  // threads per value column in the substitutions
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63;
  const int nsl = a.dv / DVS;
  const long bh = blockIdx.x / nsl;
  const int col0 = (blockIdx.x % nsl) * DVS;
  const int T = a.T, dv = a.dv;
  const int nch = (T + CH - 1) / CH;
  const long tok0 = bh * T;

  // chunk c into LDS: k, w (and q), the decay; x holds v (forward) or dO
  // (reverse); rows past the end are zero
  auto stage = [&](int c, bool with_q, const void* xsrc) {
    const int t0 = c * CH, n = min(CH, T - t0);
    if constexpr (CHAN) {
      // per channel: G_t = sum of log alpha through t (padding: alpha = 1)
      if (tid < DK) {
        const int d = tid;
        float G = 0.f;
        for (int t = 0; t < CH; ++t) {
          if (t < n) G += logf(ld<E>(a.g.alpha, (tok0 + t0 + t) * DK + d));
          sm.Gc[t * PG + d] = G;
        }
        const float gr = expf(sm.Gc[RT * PG + d]), gt = expf(G - sm.Gc[RT * PG + d]);
        sm.gref[d] = gr >= 0x1p-96f && gt >= 0x1p-96f ? gr : __builtin_nanf("");
        sm.gnr[d] = gt;
        sm.endc[d] = 0.f;
      }
      __syncthreads();
    }
    for (int idx = tid; idx < CH * DK; idx += NT) {
      const int t = idx / DK, d = idx % DK;
      const bool ok = t < n;
      const long gi = (tok0 + t0 + t) * DK + d;
      float kv = ok ? ld<E>(a.k, gi) : 0.f, wv = ok ? a.w[gi] : 0.f;
      float qv = with_q && ok ? ld<E>(a.q, gi) : 0.f;
      if constexpr (CHAN) {
        const float gd = sm.Gc[t * PG + d] - sm.Gc[RT * PG + d];
        const float ek = expf(gd);
        kv *= ek;
        qv *= ek;
        wv *= expf(-gd);
      }
      sm.k[t * PK + d] = Elem<E>::put(kv);
      sm.w[t * PK + d] = Elem<E>::put(wv);
      if (with_q) sm.q[t * PK + d] = Elem<E>::put(qv);
    }
    for (int idx = tid; idx < CH * DVS; idx += NT) {
      const int t = idx / DVS, cc = idx % DVS;
      sm.x[t * PS + cc] = t < n ? ld<E>(xsrc, (tok0 + t0 + t) * dv + col0 + cc) : 0.f;
    }
    if constexpr (!CHAN) {
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
    }
  };
  auto dotkw = [&](const E* rows, int j, int i) {  // rows_j . w_i over DK
    float s = 0.f;
#pragma unroll 8
    for (int d = 0; d < DK; ++d) s = fmaf(Elem<E>::get(rows[j * PK + d]), Elem<E>::get(sm.w[i * PK + d]), s);
    return s;
  };
  // the decay between token i and token j (scalar decay; with channel decay
  // the staged operands carry it)
  auto dec = [&](int j, int i) { return CHAN ? 1.f : expf(sm.G[j] - sm.G[i]); };
  // exp(G_t - G_r) of channel d
  auto eref = [&](int t, int d) { return expf(sm.Gc[t * PG + d] - sm.Gc[RT * PG + d]); };
  // the sum of s over the TPC threads of one value column
  auto column_sum = [&](float s) {
#pragma unroll
    for (int o = 1; o < TPC; o <<= 1) s += __shfl_xor(s, o);
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
      sm.lm[j * PC + i] = i < j && j < n ? dec(j, i) * dotkw(sm.k, j, i) : 0.f;
    }
    for (int idx = tid; idx < CH * DVS; idx += NT) {
      const int t = idx / DVS, cc = idx % DVS;
      float s = 0.f;
      for (int d = 0; d < DK; ++d) {
        const float kv = Elem<E>::get(sm.k[t * PK + d]);
        s = fmaf(CHAN ? kv * sm.gref[d] : kv, sm.S[d * PS + cc], s);
      }
      sm.x[t * PS + cc] -= CHAN ? s : sm.gam[t] * s;
    }
    __syncthreads();
    // (I + L) E = R by forward substitution, in place
    {
      const int cc = tid / TPC, part = tid % TPC;
      for (int j = 1; j < n; ++j) {
        float s = 0.f;
        for (int i = part; i < j; i += TPC) s = fmaf(sm.lm[j * PC + i], sm.x[i * PS + cc], s);
        s = column_sum(s);
        if (part == 0) sm.x[j * PS + cc] -= s;
        __syncthreads();
      }
    }
    for (int idx = tid; idx < CH * DVS; idx += NT) {
      const int t = idx / DVS, cc = idx % DVS;
      if (t < n) a.E[(tok0 + t0 + t) * dv + col0 + cc] = sm.x[t * PS + cc];
    }
    // S_out = g_n S_in + sum_t (g_n / g_t) w_t E_t^T
    const float gn = CHAN ? 1.f : sm.gam[CH - 1];
    for (int idx = tid; idx < DK * DVS; idx += NT) {
      const int d = idx / DVS, cc = idx % DVS;
      float s = 0.f;
      for (int t = 0; t < n; ++t) {
        const float wv = Elem<E>::get(sm.w[t * PK + d]);
        s = fmaf(CHAN ? wv : gn / sm.gam[t] * wv, sm.x[t * PS + cc], s);
      }
      if constexpr (CHAN)
        sm.S[d * PS + cc] = sm.gnr[d] * fmaf(sm.gref[d], sm.S[d * PS + cc], s);
      else
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
    const float gn = CHAN ? 1.f : sm.gam[CH - 1];
    // L and M
    for (int idx = tid; idx < CH * CH; idx += NT) {
      const int j = idx / CH, i = idx % CH;
      const bool in = j < n;
      const float dm = dec(j, i);
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
      for (int d = 0; d < DK; ++d) {
        const float wv = Elem<E>::get(sm.w[i * PK + d]);
        s2 = fmaf(CHAN ? wv * sm.gnr[d] : wv, sm.dS[d * PS + cc], s2);
      }
      sm.y[i * PS + cc] = i < n ? fmaf(CHAN ? 1.f : gn / sm.gam[i], s2, s) : 0.f;
    }
    // dL/dG of the chunk end: g_n <S_in, dS_out> (per channel: row d)
    if constexpr (CHAN) {
      if (tid < DK) {
        const int d = tid;
        float s = 0.f;
        for (int cc = 0; cc < DVS; ++cc) s = fmaf(sm.S[d * PS + cc], sm.dS[d * PS + cc], s);
        sm.endc[d] += sm.gref[d] * sm.gnr[d] * s;
      }
    } else {
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
      const int cc = tid / TPC, part = tid % TPC;
      for (int j = n - 2; j >= 0; --j) {
        float s = 0.f;
        for (int i = j + 1 + part; i < n; i += TPC) s = fmaf(sm.lm[i * PC + j], sm.y[i * PS + cc], s);
        s = column_sum(s);
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
    // their decay terms go to dL/dG
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
        const float kv = Elem<E>::get(sm.k[t * PK + d]), qv = Elem<E>::get(sm.q[t * PK + d]);
        const float wv = Elem<E>::get(sm.w[t * PK + d]);
        if constexpr (CHAN) {
          // g_t = exp(G_r) exp(G_t - G_r); g_n / g_t = exp(G_n - G_r) exp(G_r - G_t)
          const float er = eref(t, d), gr = sm.gref[d], gt = sm.gnr[d];
          atomicAdd(&a.dk_out[gi], gr * er * kh);
          atomicAdd(&a.dq_out[gi], gr * er * qh);
          atomicAdd(&a.dw_acc[gi], gt / er * tw);
          const float wtw = gt * wv * tw;
          atomicAdd(&a.dG[gi], gr * (kv * kh + qv * qh) - wtw);
          atomicAdd(&sm.endc[d], wtw);
        } else {
          const float g = sm.gam[t], f = gn / g;
          atomicAdd(&a.dk_out[gi], g * kh);
          atomicAdd(&a.dq_out[gi], g * qh);
          atomicAdd(&a.dw_acc[gi], f * tw);
          const float wtw = f * wv * tw;
          atomicAdd(&sm.sg[t], g * (kv * kh + qv * qh) - wtw);
          atomicAdd(&sm.sg[CH - 1], wtw);
        }
      }
    }
    __syncthreads();
    // the chunk end's dL/dG per channel is complete
    if constexpr (CHAN) {
      if (tid < DK) atomicAdd(&a.dG[(tok0 + t0 + n - 1) * DK + tid], sm.endc[tid]);
    }
    // dS_in = g_n dS_out + sum_t g_t (q_t dO_t^T - k_t dR_t^T)
    for (int idx = tid; idx < DK * DVS; idx += NT) {
      const int d = idx / DVS, cc = idx % DVS;
      float s = 0.f;
      for (int t = 0; t < n; ++t)
        s = fmaf(CHAN ? 1.f : sm.gam[t],
                 Elem<E>::get(sm.q[t * PK + d]) * sm.x[t * PS + cc] -
                     Elem<E>::get(sm.k[t * PK + d]) * sm.y[t * PS + cc],
                 s);
      if constexpr (CHAN)
        sm.dS[d * PS + cc] = sm.gref[d] * fmaf(sm.gnr[d], sm.dS[d * PS + cc], s);
      else
        sm.dS[d * PS + cc] = fmaf(gn, sm.dS[d * PS + cc], s);
    }
    // dL = -dR E^T, dM = dO E^T.  Scalar decay: their decay terms (L o dL,
    // M o dM: + to the row token, - to the column token), then L <- D o dL,
    // M <- D o dM.  Channel decay: L <- dL, M <- dM (the decay terms follow
    // per channel below)
    for (int idx = tid; idx < CH * CH; idx += NT) {
      const int j = idx / CH, i = idx % CH;
      if (j >= n || i > j) continue;
      float dl = 0.f, dmv = 0.f;
      for (int cc = 0; cc < DVS; ++cc) {
        const float ev = sm.e[i * PS + cc];
        dl = fmaf(-sm.y[j * PS + cc], ev, dl);
        dmv = fmaf(sm.x[j * PS + cc], ev, dmv);
      }
      if constexpr (CHAN) {
        sm.lm[j * PC + i] = i < j ? dl : 0.f;
        sm.mm[j * PC + i] = dmv;
      } else {
        const float dm = expf(sm.G[j] - sm.G[i]);
        const float tl = i < j ? sm.lm[j * PC + i] * dl : 0.f, tm = sm.mm[j * PC + i] * dmv;
        if (i < j) {
          atomicAdd(&sm.sg[j], tl + tm);
          atomicAdd(&sm.sg[i], -(tl + tm));
        }
        sm.lm[j * PC + i] = i < j ? dm * dl : 0.f;
        sm.mm[j * PC + i] = dm * dmv;
      }
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
      if constexpr (CHAN) {
        const float er = eref(t, d);
        atomicAdd(&a.dk_out[gi], er * sk);
        atomicAdd(&a.dq_out[gi], er * sq);
        atomicAdd(&a.dw_acc[gi], sw / er);
        atomicAdd(&a.dG[gi], Elem<E>::get(sm.k[t * PK + d]) * sk + Elem<E>::get(sm.q[t * PK + d]) * sq -
                                 Elem<E>::get(sm.w[t * PK + d]) * sw);
      } else {
        atomicAdd(&a.dk_out[gi], sk);
        atomicAdd(&a.dq_out[gi], sq);
        atomicAdd(&a.dw_acc[gi], sw);
      }
    }
    // scalar decay: dL/dG of the chunk to HBM; the padding tokens of a
    // partial chunk share the last real token's decay
    if constexpr (!CHAN) {
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
template <typename E, int DK, int GAIN, bool CHAN>
__global__ __launch_bounds__(DK) void gain_bwd_kernel(GainBwdArgs a) {
  constexpr int NW = DK / 64;
  constexpr bool PG = GAIN == GAIN_PGDN, KD = GAIN == GAIN_KDN, ISO = GAIN == GAIN_KDN_ISO;
  constexpr bool ST = PG || KD;  // a per-channel statistic, recomputed per chunk
  __shared__ float red[4][NW];
  __shared__ float As[ST ? CH : 1][ST ? DK : 1];    // PGDN: A_t; KDN: p before token t
  __shared__ float iso[ISO ? 3 : 1][ISO ? CH : 1];  // KDN_ISO: b before token t, a_t, ||k_t||^2
  const int d = threadIdx.x, wave = d >> 6, lane = d & 63;
  const long bh = blockIdx.x;
  const int h = static_cast<int>(bh % a.H);
  const int T = a.T, nch = (T + CH - 1) / CH;
  const E* kp = static_cast<const E*>(a.k);
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
  // the decay of token ti (of channel d)
  auto alpha_at = [&](long ti) {
    if constexpr (CHAN) return Elem<E>::get(static_cast<const E*>(a.g.alpha)[ti * DK + d]);
    else return static_cast<const float*>(a.g.alpha)[ti];
  };
  // dL/d(statistic after the current token), carried backwards: per channel
  // (PGDN A, KDN p) or per head (KDN_ISO b)
  float dA = 0.f;
  if (a.daux_T) {
    if constexpr (ST) dA = a.daux_T[bh * DK + d];
    if constexpr (ISO) dA = a.daux_T[bh];
  }
  float dmu = 0.f;
  const float mu = PG ? a.g.mu_log[h] : 0.f;
  const float lnx = PG ? a.g.log2x * 0.69314718055994531f : 0.f;
  const float mi = a.g.mu_info;
  for (int c = nch - 1; c >= 0; --c) {
    const int t0 = c * CH, n = min(CH, T - t0);
    if constexpr (PG) {
      // the statistic of the chunk's tokens, from its value at the chunk start
      __syncthreads();
      float A = a.aux_chunk[(bh * nch + c) * DK + d];
      for (int j = 0; j < n; ++j) {
        const long ti = bh * T + t0 + j;
        const float kk = Elem<E>::get(kp[ti * DK + d]);
        A = fmaf(a.g.alphaP[ti], A, a.g.betaP[ti] * kk * kk);
        As[j][d] = A;
      }
    } else if constexpr (KD) {
      // p before every token of the chunk: p_hat = a^2 p + omega,
      // p <- p_hat / (1 + (mu / r) k^2 p_hat)
      __syncthreads();
      float p = a.aux_chunk[(bh * nch + c) * DK + d];
      for (int j = 0; j < n; ++j) {
        const long ti = bh * T + t0 + j;
        As[j][d] = p;
        const float kk = Elem<E>::get(kp[ti * DK + d]), al = alpha_at(ti);
        const float ph = fmaf(al * al, p, Elem<E>::get(static_cast<const E*>(a.g.omega)[ti * DK + d]));
        p = ph / fmaf(mi / a.g.r[ti] * kk * kk, ph, 1.f);
      }
    } else if constexpr (ISO) {
      // b before every token, the decay's mean square a_t and ||k_t||^2
      float b = a.aux_chunk[bh * nch + c];
      for (int j = 0; j < n; ++j) {
        const long ti = bh * T + t0 + j;
        const float kk = Elem<E>::get(kp[ti * DK + d]), al = alpha_at(ti);
        float n2 = kk * kk, s2 = CHAN ? al * al : 0.f, z0 = 0.f, z1 = 0.f;
        reduce4(n2, s2, z0, z1);
        const float a2 = CHAN ? s2 / DK : al * al;
        if (d == 0) {
          iso[0][j] = b;
          iso[1][j] = a2;
          iso[2][j] = n2;
        }
        const float bh_ = fmaf(a2, b, static_cast<const float*>(a.g.omega)[ti]);
        b = bh_ / fmaf(mi * n2 / (DK * a.g.r[ti]), bh_, 1.f);
      }
    }
    __syncthreads();
    float sfx = 0.f;  // dL/d log(alpha) summed from the chunk end
    for (int j = n - 1; j >= 0; --j) {
      const long ti = bh * T + t0 + j;
      const float kk = Elem<E>::get(kp[ti * DK + d]);
      const float dw = a.dw_acc[ti * DK + d];
      float dkv = a.dk_out[ti * DK + d];
      float dag = 0.f;  // the decay's gradient through the gain (this channel's,
                        // or summed over channels for scalar decay)
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
      } else if constexpr (KD) {
        // p_hat = a^2 p + omega;  z = sum p_hat k^2;  D = r + z;  w = p_hat k / D;
        // u = (mu / r) k^2;  p_t = p_hat / (1 + u p_hat)
        const float pp = As[j][d], al = alpha_at(ti), rt = a.g.r[ti];
        const float ph = fmaf(al * al, pp, Elem<E>::get(static_cast<const E*>(a.g.omega)[ti * DK + d]));
        const float k2 = kk * kk, mr = mi / rt;
        const float gg = fmaf(mr * k2, ph, 1.f), igg2 = 1.f / (gg * gg);
        const float du = -dA * ph * ph * igg2;  // dL/du through p_t
        float z = ph * k2, dz = dw * ph * kk, duk = du * k2, z0 = 0.f;
        reduce4(z, dz, duk, z0);
        const float iD = 1.f / (rt + z);
        const float dD = -dz * iD * iD;
        const float dph = dw * kk * iD + dD * k2 + dA * igg2;
        dkv += dw * ph * iD + 2.f * kk * (dD * ph + du * mr);
        if (d == 0) a.dr[ti] = dD - duk * mr / rt;
        a.domega[ti * DK + d] = dph;
        dag = 2.f * dph * al * pp;
        dA = dph * al * al;
        if constexpr (!CHAN) {
          float z1 = 0.f, z2 = 0.f, z3 = 0.f;
          reduce4(dag, z1, z2, z3);
        }
      } else if constexpr (ISO) {
        // a = mean a_i^2;  b_hat = a b + omega;  n = ||k||^2;  beta = b_hat / (r + b_hat n);
        // w = beta k;  u = mu n / (d_k r);  b_t = b_hat / (1 + u b_hat)
        const float bp = iso[0][j], a2 = iso[1][j], n2 = iso[2][j], rt = a.g.r[ti];
        const float bh_ = fmaf(a2, bp, static_cast<const float*>(a.g.omega)[ti]);
        const float iden = 1.f / fmaf(bh_, n2, rt);
        const float beta = bh_ * iden, u = mi * n2 / (DK * rt);
        float db = dw * kk, z0 = 0.f, z1 = 0.f, z2 = 0.f;
        reduce4(db, z0, z1, z2);
        dkv = fmaf(beta, dw, dkv);
        float dbh = db * rt * iden * iden;
        float drt = -db * bh_ * iden * iden;
        float dn = -db * bh_ * bh_ * iden * iden;
        const float gg = fmaf(u, bh_, 1.f), igg2 = 1.f / (gg * gg);
        dbh += dA * igg2;
        const float du = -dA * bh_ * bh_ * igg2;
        dn += du * mi / (DK * rt);
        drt -= du * u / rt;
        dkv = fmaf(2.f * dn, kk, dkv);
        if (d == 0) {
          a.domega[ti] = dbh;
          a.dr[ti] = drt;
        }
        const float al = alpha_at(ti);
        dag = CHAN ? dbh * bp * 2.f * al / DK : dbh * bp * 2.f * al;
        dA = dbh * a2;
      }
      a.dk_out[ti * DK + d] = dkv;
      // dL/dalpha_t = (sum of dL/dG_j over j >= t in the chunk) / alpha_t,
      // plus the gain's part
      if constexpr (CHAN) {
        sfx += a.dG[ti * DK + d];
        a.dalpha[ti * DK + d] = sfx / alpha_at(ti) + dag;
      } else {
        sfx += a.dG[ti];
        if (d == 0) a.dalpha[ti] = sfx / alpha_at(ti) + dag;
      }
    }
  }
  if constexpr (ST) {
    if (a.daux0) a.daux0[bh * DK + d] = dA;
  }
  if constexpr (ISO) {
    if (a.daux0 && d == 0) a.daux0[bh] = dA;
  }
  if constexpr (PG) {
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

template <typename E, int DK, bool CHAN>
static hipError_t launch_bwd_state_t(const BwdArgs& a, hipStream_t st) {
  using Sm = bwd::Smem<E, DK, CHAN>;
  static_assert(sizeof(Sm) <= 160 * 1024, "LDS budget");
  if (a.dv % Sm::DVS != 0) return hipErrorInvalidValue;
  auto kern = bwd::chunk_bwd_state_kernel<E, DK, CHAN>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(sizeof(Sm)));
  if (err != hipSuccess) return err;
  const unsigned grid = static_cast<unsigned>(static_cast<long>(a.B) * a.H * (a.dv / Sm::DVS));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(bwd::NT), sizeof(Sm), st, a);
  return hipGetLastError();
}

template <bool CHAN>
static hipError_t launch_bwd_state_c(const BwdArgs& a, int io_bf16, hipStream_t st) {
  if (io_bf16)
    return a.dk == 128 ? launch_bwd_state_t<uint16_t, 128, CHAN>(a, st)
                       : launch_bwd_state_t<uint16_t, 64, CHAN>(a, st);
  if (a.dk == 64) return launch_bwd_state_t<float, 64, CHAN>(a, st);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_bwd_state(const BwdArgs& a, int io_bf16, bool channel, hipStream_t st) {
  if (a.T == 0 || a.B * a.H == 0) return hipSuccess;
  return channel ? launch_bwd_state_c<true>(a, io_bf16, st) : launch_bwd_state_c<false>(a, io_bf16, st);
}

template <typename E, int DK, bool CHAN>
static hipError_t launch_gain_bwd_t(const GainBwdArgs& a, int gain, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.B * a.H)), block(DK);
  switch (gain) {
#define DN_GAIN_BWD_CASE(G)                                                               \
  case G:                                                                                 \
    hipLaunchKernelGGL((bwd::gain_bwd_kernel<E, DK, G, CHAN>), grid, block, 0, st, a); \
    break;
    DN_GAIN_BWD_CASE(GAIN_KLA)
    DN_GAIN_BWD_CASE(GAIN_GDN)
    DN_GAIN_BWD_CASE(GAIN_PGDN)
    DN_GAIN_BWD_CASE(GAIN_KDN)
    DN_GAIN_BWD_CASE(GAIN_EXPLICIT)
    DN_GAIN_BWD_CASE(GAIN_KDN_ISO)
#undef DN_GAIN_BWD_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool CHAN>
static hipError_t launch_gain_bwd_c(const GainBwdArgs& a, int io_bf16, int gain, hipStream_t st) {
  if (io_bf16)
    return a.dk == 128 ? launch_gain_bwd_t<uint16_t, 128, CHAN>(a, gain, st)
                       : launch_gain_bwd_t<uint16_t, 64, CHAN>(a, gain, st);
  if (a.dk == 64) return launch_gain_bwd_t<float, 64, CHAN>(a, gain, st);
  return hipErrorInvalidValue;
}

hipError_t launch_gain_bwd(const GainBwdArgs& a, int io_bf16, int gain, bool channel,
                           hipStream_t st) {
  if (a.T == 0 || a.B * a.H == 0) return hipSuccess;
  return channel ? launch_gain_bwd_c<true>(a, io_bf16, gain, st)
                 : launch_gain_bwd_c<false>(a, io_bf16, gain, st);
}

hipError_t launch_zero(float* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(bwd::zero_kernel, dim3(static_cast<unsigned>(blocks < 4096 ? blocks : 4096)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace dn
