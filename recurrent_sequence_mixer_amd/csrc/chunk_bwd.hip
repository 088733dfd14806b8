// The split backward (bf16 io, scalar decay, after the forward chunk kernel
// has written S_ck and E).  Three launches: chunk_bwd_zp_kernel takes every
// chunk at once and forms what of (I + L)^T dR = M^T dO + W~ dS_out does not
// depend on dS (Z = (I + L)^-T W~ and P = (I + L)^-T M^T dO, so that
// dR = P + Z dS_out); chunk_bwd_ds_kernel walks the chunks from the last
// carrying dS (dR, dS_in) and stores dS_out of every chunk;
// chunk_bwd_tiles_kernel then takes every chunk at once, one workgroup per
// (b, h, chunk), and forms the per-(token, key channel) gradients dq, dk, dw
// and dL/dG from dR, dO, E, S_in and dS_out over all value columns: each is
// written once, with no atomic accumulation.

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
// chunk_bwd_state_kernel: one workgroup per (batch, head, DVS = 16 or 32
// value columns).  The value columns of dS evolve independently, so each
// workgroup carries its slice of dS; the per-token key-side gradients (dq,
// dk, dw, dG) are sums over value columns and are accumulated over the
// slices with fp32 atomics.  A forward sweep first stores the state entering
// every chunk and the residuals E (or, with BwdArgs::ck_given, the chunked
// forward's kernel has stored them); the reverse sweep then walks the chunks
// from the last.  Operands are staged in LDS (k, q, w in the io dtype, w
// rounded to it).  With fp32 io every product runs on fp32 matrix
// instructions; with bf16 io on bf16 ones, each fp32 operand as a pair of
// bf16 (hi, lo) so that the products keep nearly fp32 accuracy (mm_bf).
//
// gain_bwd_kernel (the gains with a statistic): one workgroup per (batch,
// head), one thread per key channel, walking the tokens backwards: the write
// gain's derivative (PGDN: Preconditioned DeltaNet §2.4, Eq. 9; KDN: Kalman
// Delta Networks §2.4, Eqs. 23-30 with the information scaling of §2.5;
// isotropic KDN: §2.7, Eq. 40 - the gain scan differentiated backwards,
// Appendix D), the statistic recomputed per chunk from its value at the
// chunk start, and the decay's gradient from dG.  gain_bwd_tok_kernel (KLA /
// GDN: Kaczmarz Linear Attention §2.1; explicit w): one workgroup per chunk,
// token-parallel.
#include "common.hpp"
#include "gains.hpp"
#include "launch.hpp"

namespace dn {

namespace bwd {

constexpr int CH = 64;      // chunk length
constexpr int NT = 512;     // threads of the state kernel
constexpr int NW = NT / 64; // its wavefronts
// row pitch of [CH][CH] fp32 arrays: a multiple of 4, so that four consecutive
// entries are one aligned 16-byte read, and rows four apart are 16 banks apart
constexpr int PC = CH + 4;
constexpr int PT = 17;      // row pitch of the 16x16 diagonal-block inverses
constexpr int RT = 31;      // reference token of the per-channel decay factors

// DVS_: value columns per workgroup, 16 or 32 (channel decay: 16)
template <typename E, int DK, bool CHAN, int DVS_>
struct Smem {
  static constexpr int DVS = DVS_;            // value columns per workgroup
  static constexpr int PS = DVS + 4;          // row pitch of [x][DVS] fp32 arrays (as PC)
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
  float tb[4 * 16 * PT];  // (I + L_bb)^-1 of the four diagonal 16x16 blocks
  // channel decay: G per (token, channel), exp(G_r), exp(G_n - G_r), and
  // dL/dG of the chunk's last token per channel
  float Gc[CHAN ? CH * PG : 1];
  float gref[CHAN ? DK : 1], gnr[CHAN ? DK : 1], endc[CHAN ? DK : 1];
  // scalar decay: G, exp(G), exp(G_n - G) and this slice's part of dL/dG
  // per token
  float G[CH], gam[CH], fn[CH], sg[CH];
};

template <typename E>
__device__ __forceinline__ float ld(const void* p, long i) {
  return Elem<E>::get(static_cast<const E*>(p)[i]);
}

// N consecutive elements from element offset `off` of `base` as fp32, in
// 16-byte (or 8- / 4-byte) loads; zeros when !ok.
template <typename E, int N>
__device__ __forceinline__ void load_vec(const void* base, long off, bool ok, float (&v)[N]) {
  if constexpr (sizeof(E) == 2) {
    const uint16_t* p = static_cast<const uint16_t*>(base) + off;
    uint32_t u[N / 2];
    if constexpr (N % 8 == 0) {
#pragma unroll
      for (int i = 0; i < N / 8; ++i) {
        const u32x4 x = ok ? reinterpret_cast<const u32x4*>(p)[i] : u32x4{0u, 0u, 0u, 0u};
        u[4 * i] = x[0], u[4 * i + 1] = x[1], u[4 * i + 2] = x[2], u[4 * i + 3] = x[3];
      }
    } else if constexpr (N == 4) {
      const u32x2 x = ok ? *reinterpret_cast<const u32x2*>(p) : u32x2{0u, 0u};
      u[0] = x[0], u[1] = x[1];
    } else {
      static_assert(N == 2, "bf16 vector length");
      u[0] = ok ? *reinterpret_cast<const uint32_t*>(p) : 0u;
    }
#pragma unroll
    for (int i = 0; i < N / 2; ++i) {
      v[2 * i] = __uint_as_float(u[i] << 16);
      v[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  } else {
    const float* p = static_cast<const float*>(base) + off;
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int i = 0; i < N / 4; ++i) {
        const f32x4 x = ok ? reinterpret_cast<const f32x4*>(p)[i] : zero4();
        v[4 * i] = x[0], v[4 * i + 1] = x[1], v[4 * i + 2] = x[2], v[4 * i + 3] = x[3];
      }
    } else {
      static_assert(N == 2, "fp32 vector length");
      typedef float f32x2_ __attribute__((ext_vector_type(2)));
      const f32x2_ x = ok ? *reinterpret_cast<const f32x2_*>(p) : f32x2_{0.f, 0.f};
      v[0] = x[0], v[1] = x[1];
    }
  }
}

// LDS accesses of one wavefront complete in order; the fences keep the
// compiler from moving them across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Sums over the 16 lanes of a row group (lanes 16 g .. 16 g + 15) and over
// the four row groups (lanes with the same l % 16).  The row sum moves data
// by DPP (quad permutes, then the half-row and row mirrors), not through the
// LDS crossbar; every lane of the wavefront must be active.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_move<0xB1>(v);   // quad_perm(1,0,3,2)
  v += dpp_move<0x4E>(v);   // quad_perm(2,3,0,1)
  v += dpp_move<0x141>(v);  // row_half_mirror: the other quad of the 8
  v += dpp_move<0x140>(v);  // row_mirror: the other 8 of the 16
  return v;
}
// the sum over the wavefront, in every lane: row sums, then the four row
// totals read back through scalar registers (every lane active)
__device__ __forceinline__ float wave_total(float v) {
  v = row16_sum(v);
  auto rl = [&](int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); };
  return (rl(0) + rl(16)) + (rl(32) + rl(48));
}
__device__ __forceinline__ float col4_sum(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x16_bf16: lane l supplies A row l % 16 and B column l % 16
// at k = 4 (l / 16) .. +3; the result has the layout of mfma4's
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// An fp32 value as a pair of bf16, hi = bf16(v) and lo = bf16(v - hi), in one
// word (hi in the low half): hi + lo equals v to about 2^-17 of |v|, so a
// product of such a value with a bf16 value takes two bf16 matrix
// instructions at nearly fp32 accuracy.  The fp32 zero is the pair (0, 0).
__device__ __forceinline__ uint32_t split_bf(float v) {
  const uint16_t hi = f2bf(v);
  return static_cast<uint32_t>(hi) | (static_cast<uint32_t>(f2bf(v - bf2f(hi))) << 16);
}
// two bf16 in one word, a in the low half
__device__ __forceinline__ uint32_t pack16(uint16_t a, uint16_t b) {
  return static_cast<uint32_t>(a) | (static_cast<uint32_t>(b) << 16);
}
// the hi and lo halves of four split words as two bf16x4 operands
__device__ __forceinline__ void split4(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3, s16x4& hi,
                                       s16x4& lo) {
  hi = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(x1, x0, 0x05040100u),
                                       __builtin_amdgcn_perm(x3, x2, 0x05040100u)});
  lo = __builtin_bit_cast(s16x4, u32x2{__builtin_amdgcn_perm(x1, x0, 0x07060302u),
                                       __builtin_amdgcn_perm(x3, x2, 0x07060302u)});
}
// four bf16 at stride `ld` (a column of a row-major array) as one operand
__device__ __forceinline__ s16x4 bf4_col(const uint16_t* p, int ld) {
  return __builtin_bit_cast(s16x4, u32x2{static_cast<uint32_t>(p[0]) | (static_cast<uint32_t>(p[ld]) << 16),
                                         static_cast<uint32_t>(p[2 * ld]) | (static_cast<uint32_t>(p[3 * ld]) << 16)});
}
// four consecutive bf16 of a row from k (a multiple of 4; rows at a pitch of
// an even number of elements, so both halves are 4-byte aligned)
__device__ __forceinline__ s16x4 bf4(const uint16_t* row, int k) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(row + k);
  return __builtin_bit_cast(s16x4, u32x2{p[0], p[1]});
}

// One 16x16 output tile of a product on v_mfma_f32_16x16x4_f32:
// acc += sum over k in [k0, k1) of A[r][k] B[k][c], k0 and k1 multiples of 4,
// fa(r, k) = A[r][k], fb(k, c) = B[k][c] (tile-local r, c).  Lane l supplies
// A row l % 16 and B column l % 16 at k = k0 + 4 s + l / 16; on return lane l
// holds rows 4 (l / 16) + i, i = 0..3, of column l % 16.
template <typename FA, typename FB>
__device__ __forceinline__ f32x4 mm(f32x4 acc, int k0, int k1, FA fa, FB fb, int lane) {
  const int r = lane & 15, kq = lane >> 4;
#pragma unroll 4
  for (int k = k0; k < k1; k += 4) acc = mfma4(fa(r, k + kq), fb(k + kq, r), acc);
  return acc;
}

// four consecutive fp32 values from a 16-byte aligned LDS address, as one read
__device__ __forceinline__ void ld4(float (&v)[4], const float* p) {
  const f32x4 x = *reinterpret_cast<const f32x4*>(p);
  v[0] = x[0], v[1] = x[1], v[2] = x[2], v[3] = x[3];
}
// Four fp32 values as bf16 pairs: hi4 keeps the upper half of each value
// (truncation), lo4 = bf16(v - hi) (v - hi is exact in fp32); hi + lo is
// within 2^-16 of |v|.  For values that are bf16 numbers lo is zero.
__device__ __forceinline__ s16x4 hi4(const float (&v)[4]) {
  return __builtin_bit_cast(
      s16x4, u32x2{__builtin_amdgcn_perm(__float_as_uint(v[1]), __float_as_uint(v[0]), 0x07060302u),
                   __builtin_amdgcn_perm(__float_as_uint(v[3]), __float_as_uint(v[2]), 0x07060302u)});
}
__device__ __forceinline__ s16x4 lo4(const float (&v)[4]) {
  auto r = [&](int j) { return v[j] - __uint_as_float(__float_as_uint(v[j]) & 0xffff0000u); };
  return __builtin_bit_cast(s16x4, u32x2{pack_bf2(r(0), r(1)), pack_bf2(r(2), r(3))});
}
// mm on v_mfma_f32_16x16x16_bf16 with the fp32 operands as bf16 pairs:
// lo A hi B + hi A lo B + hi A hi B (the lo lo term, below 2^-32 of the
// product, is dropped).  AX / BX: the operand's values are bf16 numbers
// (k, q, w and dO with bf16 io), so its lo term is zero and skipped.  k0 and
// k1 multiples of 16; lane l supplies k = k0 + 16 s + 4 (l / 16) .. +3.
template <bool AX, bool BX, typename FA, typename FB>
__device__ __forceinline__ f32x4 mm_bf(f32x4 acc, int k0, int k1, FA fa, FB fb, int lane) {
  const int r = lane & 15, kq = lane >> 4;
#pragma unroll 1
  for (int k = k0; k < k1; k += 16) {
    float av[4], bv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      av[j] = fa(r, k + 4 * kq + j);
      bv[j] = fb(k + 4 * kq + j, r);
    }
    const s16x4 ah = hi4(av), bh = hi4(bv);
    if constexpr (!AX) acc = mfma16(lo4(av), bh, acc);
    if constexpr (!BX) acc = mfma16(ah, lo4(bv), acc);
    acc = mfma16(ah, bh, acc);
  }
  return acc;
}

template <typename E, int DK, bool CHAN, int DVS_>
__global__ __launch_bounds__(NT) void chunk_bwd_state_kernel(BwdArgs a) {
  using Sm = Smem<E, DK, CHAN, DVS_>;
  constexpr int PK = Sm::PK, PS = Sm::PS, PG = Sm::PG, DVS = Sm::DVS;
  // the fp32 arrays read as 16-byte pieces start on 16-byte boundaries
  static_assert(offsetof(Sm, S) % 16 == 0 && offsetof(Sm, dS) % 16 == 0 && offsetof(Sm, e) % 16 == 0 &&
                    offsetof(Sm, x) % 16 == 0 && offsetof(Sm, y) % 16 == 0 && offsetof(Sm, lm) % 16 == 0 &&
                    offsetof(Sm, mm) % 16 == 0 && PS % 4 == 0 && PC % 4 == 0,
                "16-byte LDS rows");
  constexpr int NC = DVS / 16;      // 16-column tiles of the value slice
  constexpr int ND = DK / 16;       // 16-row tiles of the key dimension
  constexpr int TPW = 4 * ND / NW;  // [token][key] tiles per wavefront
  static_assert(TPW * NW == 4 * ND, "key tiles per wavefront");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  DN_LDS_POISON(smem_raw, sizeof(Sm));
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;  // tile column / row group of this lane
  const int nsl = a.dv / DVS;
  const long bh = blockIdx.x / nsl;
  const int col0 = (blockIdx.x % nsl) * DVS;
  const int T = a.T, dv = a.dv;
  const int nch = (T + CH - 1) / CH;
  const long tok0 = bh * T;
  auto kf = [&](int t, int d) { return Elem<E>::get(sm.k[t * PK + d]); };
  auto qf = [&](int t, int d) { return Elem<E>::get(sm.q[t * PK + d]); };
  auto wf = [&](int t, int d) { return Elem<E>::get(sm.w[t * PK + d]); };
  // A B over k0 .. k1: bf16 io on bf16 instructions with split fp32 operands
  // (AX / BX as for mm_bf), fp32 io on fp32 instructions
  auto mmx = [&](auto ax, auto bx, f32x4 acc, int k0, int k1, auto fa, auto fb) __attribute__((always_inline)) {
    if constexpr (sizeof(E) == 2)
      return mm_bf<decltype(ax)::value, decltype(bx)::value>(acc, k0, k1, fa, fb, lane);
    else
      return mm(acc, k0, k1, fa, fb, lane);
  };
  constexpr std::true_type EXACT{};
  constexpr std::false_type SPLIT{};

  // chunk c into LDS: k, w, the decay, x = v (forward); reverse also q,
  // x = dO, the residuals e and the state entering the chunk.  Rows past the
  // end are zero.  Every thread first issues all its global loads (16-byte
  // vectors of consecutive elements), then converts and stores.
  constexpr int KV = CH * DK / NT, XV = CH * DVS / NT, SV = DK * DVS / NT;
  auto stage = [&](int c, bool rev) {
    const int t0 = c * CH, n = min(CH, T - t0);
    const int kt = tid * KV / DK, kd = tid * KV % DK;
    const int xt = tid * XV / DVS, xc = tid * XV % DVS;
    const int sd = tid * SV / DVS, sc = tid * SV % DVS;
    const long krow = (tok0 + t0 + kt) * DK + kd, xrow = (tok0 + t0 + xt) * dv + col0 + xc;
    const bool kok = kt < n, xok = xt < n;
    float kv[KV], qv[KV], wv[KV], xv[XV], ev[XV], sv[SV], av[CHAN ? KV : 1];
    load_vec<E, KV>(a.k, krow, kok, kv);
    // bf16 write vectors with bf16 io and scalar decay (already rounded as
    // they are stored below), fp32 otherwise
    if constexpr (sizeof(E) == 2 && !CHAN)
      load_vec<E, KV>(a.w, krow, kok, wv);
    else
      load_vec<float, KV>(a.w, krow, kok, wv);
    load_vec<E, XV>(rev ? a.dO : a.v, xrow, xok, xv);
    if (rev) {
      load_vec<E, KV>(a.q, krow, kok, qv);
      load_vec<float, XV>(a.E, xrow, xok, ev);
      load_vec<float, SV>(a.S_ck, ((bh * nch + c) * DK + sd) * dv + col0 + sc, true, sv);
    }
    if constexpr (CHAN) {
      load_vec<E, KV>(a.g.alpha, krow, kok, av);
      // per channel: G_t = sum of log alpha through t (padding: alpha = 1)
#pragma unroll
      for (int j = 0; j < KV; ++j) sm.Gc[kt * PG + kd + j] = kok ? logf(av[j]) : 0.f;
      __syncthreads();
      if (tid < DK) {
        const int d = tid;
        float G = 0.f, Gr = 0.f;
#pragma unroll 16
        for (int t = 0; t < CH; ++t) {
          G += sm.Gc[t * PG + d];
          sm.Gc[t * PG + d] = G;
          if (t == RT) Gr = G;
        }
        const float gr = expf(Gr), gt = expf(G - Gr);
        sm.gref[d] = gr >= 0x1p-96f && gt >= 0x1p-96f ? gr : __builtin_nanf("");
        sm.gnr[d] = gt;
        sm.endc[d] = 0.f;
      }
      __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < KV; ++j) {
      const int d = kd + j;
      float k_ = kv[j], q_ = rev ? qv[j] : 0.f, w_ = wv[j];
      if constexpr (CHAN) {
        const float gd = sm.Gc[kt * PG + d] - sm.Gc[RT * PG + d];
        const float ek = expf(gd);
        k_ *= ek;
        q_ *= ek;
        w_ *= expf(-gd);
      }
      sm.k[kt * PK + d] = Elem<E>::put(k_);
      sm.w[kt * PK + d] = Elem<E>::put(w_);
      if (rev) sm.q[kt * PK + d] = Elem<E>::put(q_);
    }
#pragma unroll
    for (int j = 0; j < XV; ++j) {
      sm.x[xt * PS + xc + j] = xv[j];
      if (rev) sm.e[xt * PS + xc + j] = ev[j];
    }
    if (rev) {
#pragma unroll
      for (int j = 0; j < SV; ++j) sm.S[sd * PS + sc + j] = sv[j];
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
        // g_n / g_t from the difference of the logs: no quotient of two
        // exponentials that may both underflow
        sm.fn[tid] = expf(__shfl(l, CH - 1) - l);
        sm.sg[tid] = 0.f;
      }
    }
  };
  // the decay between token i and token j (scalar decay; with channel decay
  // the staged operands carry it)
  auto dec = [&](int j, int i) { return CHAN ? 1.f : expf(sm.G[j] - sm.G[i]); };
  // exp(G_t - G_r) of channel d
  auto eref = [&](int t, int d) { return expf(sm.Gc[t * PG + d] - sm.Gc[RT * PG + d]); };
  // L = strict_lower(D o K W^T) (and, with_m, M = lower(D o Q W^T)) of the
  // chunk's n tokens into lm (mm); tiles above the diagonal are zero
  auto form_lm = [&](int n, bool with_m) {
    for (int tile = wave; tile < 16; tile += NW) {
      const int tr = tile >> 2, tc = tile & 3;
      f32x4 al = zero4(), am = zero4();
      if (tr >= tc && sizeof(E) == 2) {
        // bf16 operands: products of bf16 values are exact, so the bf16 matrix
        // instruction (16 k per step) gives the fp32 instruction's sums
        const uint16_t* kr = reinterpret_cast<const uint16_t*>(sm.k) + (16 * tr + lr) * PK;
        const uint16_t* qr = reinterpret_cast<const uint16_t*>(sm.q) + (16 * tr + lr) * PK;
        const uint16_t* wr = reinterpret_cast<const uint16_t*>(sm.w) + (16 * tc + lr) * PK;
#pragma unroll 4
        for (int k0 = 0; k0 < DK; k0 += 16) {
          const int k_ = k0 + 4 * lg;
          const s16x4 wv = bf4(wr, k_);
          al = mfma16(bf4(kr, k_), wv, al);
          if (with_m) am = mfma16(bf4(qr, k_), wv, am);
        }
      } else if (tr >= tc) {
        if (with_m) {
#pragma unroll 4
          for (int k0 = 0; k0 < DK; k0 += 4) {
            const int k_ = k0 + lg;
            const float wv = wf(16 * tc + lr, k_);
            al = mfma4(kf(16 * tr + lr, k_), wv, al);
            am = mfma4(qf(16 * tr + lr, k_), wv, am);
          }
        } else {
          al = mm(al, 0, DK, [&](int r, int k_) { return kf(16 * tr + r, k_); },
                  [&](int k_, int c) { return wf(16 * tc + c, k_); }, lane);
        }
      }
      const int i = 16 * tc + lr;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int j = 16 * tr + 4 * lg + ii;
        const float dm = j < n && i <= j ? dec(j, i) : 0.f;
        sm.lm[j * PC + i] = i < j ? dm * al[ii] : 0.f;
        if (with_m) sm.mm[j * PC + i] = dm * am[ii];
      }
    }
  };
  // (I + L_bb)^-1 of the diagonal blocks, by forward substitution (waves 0..3,
  // lane c holds column c)
  auto invert_blocks = [&]() {
    if (wave < 4 && lane < 16) {
      const int b = wave, c = lane;
      float t[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = r == c ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) s = fmaf(-sm.lm[(16 * b + r) * PC + 16 * b + m], t[m], s);
        t[r] = s;
        sm.tb[(16 * b + r) * PT + c] = s;
      }
    }
  };
  // block b of a solve, in place in the 16-column tile cb of X:
  // X_b <- T_b (X_b - acc) (or T_b^T when `tr`).  The product's k index runs
  // over the rows this lane holds, 4 (lane / 16) + s, matched in T_b.
  auto apply_block = [&](float* X, int b, int cb, f32x4 acc, bool tr) {
    f32x4 z, u = zero4();
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = X[(16 * b + 4 * lg + i) * PS + 16 * cb + lr] - acc[i];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float tv = tr ? sm.tb[(16 * b + 4 * lg + s) * PT + lr] : sm.tb[(16 * b + lr) * PT + 4 * lg + s];
      u = mfma4(tv, z[s], u);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) X[(16 * b + 4 * lg + i) * PS + 16 * cb + lr] = u[i];
    wave_lds_sync();
  };
  // (I + L) Z = X: Z_b = T_b (X_b - sum_{m<b} L_bm Z_m), one wave per column tile
  auto solve_lower = [&](float* X) {
    for (int cb = wave; cb < NC; cb += NW)
      for (int b = 0; b < 4; ++b) {
        const f32x4 acc = mmx(SPLIT, SPLIT, zero4(), 0, 16 * b, [&](int r, int k_) { return sm.lm[(16 * b + r) * PC + k_]; },
                              [&](int k_, int c) { return X[k_ * PS + 16 * cb + c]; });
        apply_block(X, b, cb, acc, false);
      }
  };
  // (I + L)^T Z = X: Z_b = T_b^T (X_b - sum_{m>b} L_mb^T Z_m)
  auto solve_upper = [&](float* X) {
    for (int cb = wave; cb < NC; cb += NW)
      for (int b = 3; b >= 0; --b) {
        const f32x4 acc = mmx(SPLIT, SPLIT, zero4(), 16 * (b + 1), CH, [&](int r, int k_) { return sm.lm[k_ * PC + 16 * b + r]; },
                              [&](int k_, int c) { return X[k_ * PS + 16 * cb + c]; });
        apply_block(X, b, cb, acc, true);
      }
  };

  // ---------------- forward sweep: S_in of every chunk and E
  // (skipped when the forward chunk kernel wrote the checkpoints)
  if (!a.ck_given) {
    for (int idx = tid; idx < DK * DVS; idx += NT) {
      const int d = idx / DVS, cc = idx % DVS;
      sm.S[d * PS + cc] = a.S0 ? a.S0[(bh * DK + d) * dv + col0 + cc] : 0.f;
    }
    for (int c = 0; c < nch; ++c) {
      const int t0 = c * CH, n = min(CH, T - t0);
      __syncthreads();  // the previous chunk's readers of k, w, x, S are done
      stage(c, false);
      __syncthreads();
      // S_in to the checkpoint; L; R = V - g K S_in
      for (int idx = tid; idx < DK * DVS; idx += NT) {
        const int d = idx / DVS, cc = idx % DVS;
        a.S_ck[((bh * nch + c) * DK + d) * dv + col0 + cc] = sm.S[d * PS + cc];
      }
      form_lm(n, false);
      for (int tile = wave; tile < 4 * NC; tile += NW) {
        const int tb_ = tile / NC, cb = tile % NC;
        const f32x4 acc =
            mmx(EXACT, SPLIT, zero4(), 0, DK, [&](int r, int k_) { return kf(16 * tb_ + r, k_); },
                [&](int k_, int cc) { return CHAN ? sm.gref[k_] * sm.S[k_ * PS + 16 * cb + cc] : sm.S[k_ * PS + 16 * cb + cc]; });
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int t = 16 * tb_ + 4 * lg + ii;
          sm.x[t * PS + 16 * cb + lr] -= CHAN ? acc[ii] : sm.gam[t] * acc[ii];
        }
      }
      __syncthreads();
      invert_blocks();
      __syncthreads();
      solve_lower(sm.x);  // E
      __syncthreads();
      for (int idx = tid; idx < CH * DVS; idx += NT) {
        const int t = idx / DVS, cc = idx % DVS;
        if (t < n) a.E[(tok0 + t0 + t) * dv + col0 + cc] = sm.x[t * PS + cc];
      }
      // S_out = g_n S_in + sum_t (g_n / g_t) w_t E_t^T
      const float gn = CHAN ? 1.f : sm.gam[CH - 1];
      for (int tile = wave; tile < ND * NC; tile += NW) {
        const int db = tile / NC, cb = tile % NC;
        const f32x4 acc =
            mmx(EXACT, SPLIT, zero4(), 0, CH, [&](int r, int k_) { return wf(k_, 16 * db + r); },
                [&](int k_, int cc) { return CHAN ? sm.x[k_ * PS + 16 * cb + cc] : sm.fn[k_] * sm.x[k_ * PS + 16 * cb + cc]; });
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int d = 16 * db + 4 * lg + ii;
          float& s = sm.S[d * PS + 16 * cb + lr];
          s = CHAN ? sm.gnr[d] * fmaf(sm.gref[d], s, acc[ii]) : fmaf(gn, s, acc[ii]);
        }
      }
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
    stage(c, true);
    __syncthreads();
    const float gn = CHAN ? 1.f : sm.gam[CH - 1];
    form_lm(n, true);
    __syncthreads();
    invert_blocks();
    // dE = M^T dO + W~ dS_out
    for (int tile = wave; tile < 4 * NC; tile += NW) {
      const int ib = tile / NC, cb = tile % NC;
      const f32x4 a1 = mmx(SPLIT, EXACT, zero4(), 16 * ib, CH, [&](int r, int k_) { return sm.mm[k_ * PC + 16 * ib + r]; },
                           [&](int k_, int cc) { return sm.x[k_ * PS + 16 * cb + cc]; });
      const f32x4 a2 =
          mmx(EXACT, SPLIT, zero4(), 0, DK, [&](int r, int k_) { return wf(16 * ib + r, k_); },
              [&](int k_, int cc) { return CHAN ? sm.gnr[k_] * sm.dS[k_ * PS + 16 * cb + cc] : sm.dS[k_ * PS + 16 * cb + cc]; });
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * ib + 4 * lg + ii;
        sm.y[i * PS + 16 * cb + lr] = i < n ? fmaf(CHAN ? 1.f : sm.fn[i], a2[ii], a1[ii]) : 0.f;
      }
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
      s = wave_total(s);
      if (lane == 0) atomicAdd(&sm.sg[CH - 1], gn * s);
    }
    __syncthreads();
    solve_upper(sm.y);  // dR
    __syncthreads();
    // dV = dR
    for (int idx = tid; idx < CH * DVS; idx += NT) {
      const int t = idx / DVS, cc = idx % DVS;
      if (t < n) a.dv_out[(tok0 + t0 + t) * dv + col0 + cc] = sm.y[t * PS + cc];
    }
    // dL = -dR E^T, dM = dO E^T.  Scalar decay: their decay terms (L o dL,
    // M o dM: + to the row token, - to the column token), then L <- D o dL,
    // M <- D o dM.  Channel decay: L <- dL, M <- dM (the decay terms follow
    // per channel below).  bf16 io: stored as split pairs (split_bf) for the
    // products with the bf16 operands below; the entries not written are 0
    // in either form
    auto put_lm = [&](int at, float l, float m) __attribute__((always_inline)) {
      if constexpr (sizeof(E) == 2) {
        reinterpret_cast<uint32_t*>(sm.lm)[at] = split_bf(l);
        reinterpret_cast<uint32_t*>(sm.mm)[at] = split_bf(m);
      } else {
        sm.lm[at] = l;
        sm.mm[at] = m;
      }
    };
    for (int tile = wave; tile < 16; tile += NW) {
      const int tr = tile >> 2, tc = tile & 3;
      if (tr < tc) continue;
      f32x4 al = zero4(), am = zero4();
      if constexpr (sizeof(E) == 2) {
        // as mm_bf, E split once for both products (dO is a bf16 number)
#pragma unroll
        for (int k0 = 0; k0 < DVS; k0 += 16) {
          const int k_ = k0 + 4 * lg;
          float ev[4], yv[4], xv[4];
          ld4(ev, &sm.e[(16 * tc + lr) * PS + k_]);
          ld4(yv, &sm.y[(16 * tr + lr) * PS + k_]);
          ld4(xv, &sm.x[(16 * tr + lr) * PS + k_]);
          const s16x4 eh = hi4(ev), el = lo4(ev), yh = hi4(yv), xh = hi4(xv);
          al = mfma16(yh, eh, mfma16(yh, el, mfma16(lo4(yv), eh, al)));
          am = mfma16(xh, eh, mfma16(xh, el, am));
        }
      } else {
#pragma unroll
        for (int k0 = 0; k0 < DVS; k0 += 4) {
          const int k_ = k0 + lg;
          const float ev = sm.e[(16 * tc + lr) * PS + k_];
          al = mfma4(sm.y[(16 * tr + lr) * PS + k_], ev, al);
          am = mfma4(sm.x[(16 * tr + lr) * PS + k_], ev, am);
        }
      }
      const int i = 16 * tc + lr;
      float col = 0.f;  // scalar decay: - (L o dL + M o dM) summed over this lane's rows
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int j = 16 * tr + 4 * lg + ii;
        const bool ok = j < n && i <= j;
        const float dl = -al[ii], dmv = am[ii];
        if constexpr (CHAN) {
          if (ok) {
            put_lm(j * PC + i, i < j ? dl : 0.f, dmv);
          }
        } else {
          float tlm = 0.f;
          if (ok) {
            const float dm = expf(sm.G[j] - sm.G[i]);
            tlm = (i < j ? sm.lm[j * PC + i] * dl : 0.f) + sm.mm[j * PC + i] * dmv;
            if (i == j) tlm = 0.f;  // the diagonal adds and subtracts the same term
            put_lm(j * PC + i, i < j ? dm * dl : 0.f, dm * dmv);
          }
          col -= tlm;
          const float row = row16_sum(tlm);  // + to the row token j
          if (lr == 0 && j < n) atomicAdd(&sm.sg[j], row);
        }
      }
      if constexpr (!CHAN) {
        col = col4_sum(col);  // - to the column token i
        if (lg == 0) atomicAdd(&sm.sg[i], col);
      }
    }
    __syncthreads();
    // per (token, key channel) tile, with one addition per gradient element
    // and value slice:
    //   through S_in and dS_out: dk += g_t (-S_in dR_t), dq += g_t (S_in dO_t),
    //     dw += (g_n / g_t) dS_out E_t, and their decay terms;
    //   through L and M: dk += sum_{i<t} (D o dL)_ti w_i,
    //     dq += sum_{i<=t} (D o dM)_ti w_i,
    //     dw_t += sum_{j>t} (D o dL)_jt k_j + sum_{j>=t} (D o dM)_jt q_j
    float wend = 0.f;  // scalar decay: the chunk end's part of the W~ terms
#pragma unroll 1
    for (int tile = wave; tile < 4 * ND; tile += NW) {
      const int tb_ = tile / ND, db = tile % ND;
      // the tile's products, independent chains interleaved (operands as
      // for mm: A row lr, B column lr, k = 4 s + lg)
      f32x4 akh = zero4(), aqh = zero4(), atw = zero4();
      if constexpr (sizeof(E) == 2) {
        // as mm_bf, S split once for both of its products (dO is a bf16 number)
#pragma unroll
        for (int k0 = 0; k0 < DVS; k0 += 16) {
          const int k_ = k0 + 4 * lg;
          float sv[4], dsv[4], yv[4], xv[4], ev[4];
          ld4(sv, &sm.S[(16 * db + lr) * PS + k_]);
          ld4(dsv, &sm.dS[(16 * db + lr) * PS + k_]);
          ld4(yv, &sm.y[(16 * tb_ + lr) * PS + k_]);
          ld4(xv, &sm.x[(16 * tb_ + lr) * PS + k_]);
          ld4(ev, &sm.e[(16 * tb_ + lr) * PS + k_]);
          const s16x4 sh = hi4(sv), sl = lo4(sv), dh = hi4(dsv), yh = hi4(yv), xh = hi4(xv), eh = hi4(ev);
          akh = mfma16(yh, sh, mfma16(yh, sl, mfma16(lo4(yv), sh, akh)));
          aqh = mfma16(xh, sh, mfma16(xh, sl, aqh));
          atw = mfma16(eh, dh, mfma16(eh, lo4(dsv), mfma16(lo4(ev), dh, atw)));
        }
      } else {
#pragma unroll
        for (int k0 = 0; k0 < DVS; k0 += 4) {
          const int k_ = k0 + lg;
          const float sv = sm.S[(16 * db + lr) * PS + k_];
          akh = mfma4(sm.y[(16 * tb_ + lr) * PS + k_], sv, akh);
          aqh = mfma4(sm.x[(16 * tb_ + lr) * PS + k_], sv, aqh);
          atw = mfma4(sm.e[(16 * tb_ + lr) * PS + k_], sm.dS[(16 * db + lr) * PS + k_], atw);
        }
      }
      f32x4 ask = zero4(), asq = zero4(), asw = zero4(), asw2 = zero4();
      if constexpr (sizeof(E) == 2) {
        // (D o dL), (D o dM) as split pairs times the bf16 w, k, q: two bf16
        // matrix instructions per 16 k
        const uint32_t* lmu = reinterpret_cast<const uint32_t*>(sm.lm);
        const uint32_t* mmu = reinterpret_cast<const uint32_t*>(sm.mm);
        const uint16_t* wb = reinterpret_cast<const uint16_t*>(sm.w) + 16 * db + lr;
        const uint16_t* kb = reinterpret_cast<const uint16_t*>(sm.k) + 16 * db + lr;
        const uint16_t* qb = reinterpret_cast<const uint16_t*>(sm.q) + 16 * db + lr;
#pragma unroll 2
        for (int k0 = 0; k0 < 16 * (tb_ + 1); k0 += 16) {
          const int k_ = k0 + 4 * lg;
          const s16x4 wv = bf4_col(wb + k_ * PK, PK);
          const u32x4 lw = *reinterpret_cast<const u32x4*>(lmu + (16 * tb_ + lr) * PC + k_);
          const u32x4 mw = *reinterpret_cast<const u32x4*>(mmu + (16 * tb_ + lr) * PC + k_);
          s16x4 h, l;
          split4(lw[0], lw[1], lw[2], lw[3], h, l);
          ask = mfma16(l, wv, mfma16(h, wv, ask));
          split4(mw[0], mw[1], mw[2], mw[3], h, l);
          asq = mfma16(l, wv, mfma16(h, wv, asq));
        }
#pragma unroll 2
        for (int k0 = 16 * tb_; k0 < CH; k0 += 16) {
          const int k_ = k0 + 4 * lg;
          const uint32_t* lc = lmu + k_ * PC + 16 * tb_ + lr;
          const uint32_t* mc = mmu + k_ * PC + 16 * tb_ + lr;
          s16x4 h, l;
          split4(lc[0], lc[PC], lc[2 * PC], lc[3 * PC], h, l);
          const s16x4 kv = bf4_col(kb + k_ * PK, PK);
          asw = mfma16(l, kv, mfma16(h, kv, asw));
          split4(mc[0], mc[PC], mc[2 * PC], mc[3 * PC], h, l);
          const s16x4 qv = bf4_col(qb + k_ * PK, PK);
          asw2 = mfma16(l, qv, mfma16(h, qv, asw2));
        }
      } else {
#pragma unroll 4
        for (int k0 = 0; k0 < 16 * (tb_ + 1); k0 += 4) {
          const int k_ = k0 + lg;
          const float wv = wf(k_, 16 * db + lr);
          ask = mfma4(sm.lm[(16 * tb_ + lr) * PC + k_], wv, ask);
          asq = mfma4(sm.mm[(16 * tb_ + lr) * PC + k_], wv, asq);
        }
#pragma unroll 4
        for (int k0 = 16 * tb_; k0 < CH; k0 += 4) {
          const int k_ = k0 + lg;
          asw = mfma4(sm.lm[k_ * PC + 16 * tb_ + lr], kf(k_, 16 * db + lr), asw);
          asw2 = mfma4(sm.mm[k_ * PC + 16 * tb_ + lr], qf(k_, 16 * db + lr), asw2);
        }
      }
      asw += asw2;
      float ce = 0.f;  // channel decay: this lane's part of the chunk end's dL/dG
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int t = 16 * tb_ + 4 * lg + ii, d = 16 * db + lr;
        const bool ok = t < n;
        const long gi = (tok0 + t0 + t) * DK + d;
        const float kh = -akh[ii], qh = aqh[ii], tw = atw[ii];
        const float sk = ask[ii], sq = asq[ii], sw = asw[ii];
        const float kv = kf(t, d), qv = qf(t, d), wv = wf(t, d);
        if constexpr (CHAN) {
          // g_t = exp(G_r) exp(G_t - G_r); g_n / g_t = exp(G_n - G_r) exp(G_r - G_t)
          const float er = eref(t, d), gr = sm.gref[d], gt = sm.gnr[d];
          const float wtw = gt * wv * tw;
          if (ok) {
            atomicAdd(&a.dk_out[gi], er * fmaf(gr, kh, sk));
            atomicAdd(&a.dq_out[gi], er * fmaf(gr, qh, sq));
            atomicAdd(&a.dw_acc[gi], fmaf(gt, tw, sw) / er);
            atomicAdd(&a.dG[gi], gr * (kv * kh + qv * qh) - wtw + kv * sk + qv * sq - wv * sw);
            ce += wtw;
          }
        } else {
          const float g = sm.gam[t], f = sm.fn[t];
          const float wtw = f * wv * tw;
          if (ok) {
            atomicAdd(&a.dk_out[gi], fmaf(g, kh, sk));
            atomicAdd(&a.dq_out[gi], fmaf(g, qh, sq));
            atomicAdd(&a.dw_acc[gi], fmaf(f, tw, sw));
            wend += wtw;
          }
          const float row = row16_sum(ok ? g * (kv * kh + qv * qh) - wtw : 0.f);
          if (lr == 0 && ok) atomicAdd(&sm.sg[t], row);
        }
      }
      if constexpr (CHAN) {
        ce = col4_sum(ce);
        if (lg == 0) atomicAdd(&sm.endc[16 * db + lr], ce);
      }
    }
    if constexpr (!CHAN) {
      wend = wave_total(wend);
      if (lane == 0) atomicAdd(&sm.sg[CH - 1], wend);
    }
    __syncthreads();
    // the chunk end's dL/dG per channel is complete
    if constexpr (CHAN) {
      if (tid < DK) atomicAdd(&a.dG[(tok0 + t0 + n - 1) * DK + tid], sm.endc[tid]);
    }
    // dS_in = g_n dS_out + sum_t g_t (q_t dO_t^T - k_t dR_t^T)
    for (int tile = wave; tile < ND * NC; tile += NW) {
      const int db = tile / NC, cb = tile % NC;
      auto gk = [&](int k_) { return CHAN ? 1.f : sm.gam[k_]; };
      f32x4 acc = mmx(EXACT, SPLIT, zero4(), 0, CH, [&](int r, int k_) { return qf(k_, 16 * db + r); },
                      [&](int k_, int cc) { return gk(k_) * sm.x[k_ * PS + 16 * cb + cc]; });
      const f32x4 acc2 = mmx(EXACT, SPLIT, zero4(), 0, CH, [&](int r, int k_) { return kf(k_, 16 * db + r); },
                             [&](int k_, int cc) { return gk(k_) * sm.y[k_ * PS + 16 * cb + cc]; });
      acc -= acc2;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int d = 16 * db + 4 * lg + ii;
        float& s = sm.dS[d * PS + 16 * cb + lr];
        s = CHAN ? sm.gref[d] * fmaf(sm.gnr[d], s, acc[ii]) : fmaf(gn, s, acc[ii]);
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
// The split backward (bf16 io, scalar decay, after the forward chunk kernel
// has written S_ck and E).  chunk_bwd_ds_kernel walks the chunks from the
// last doing only what carries dS: dE = M^T dO + W~ dS_out, dR from
// (I + L)^T dR = dE (written as dV), and dS_in; it stores dS_out of every
// chunk.  chunk_bwd_tiles_kernel then takes every chunk at once, one
// workgroup per (b, h, chunk), and forms the per-(token, key channel)
// gradients dq, dk, dw and dL/dG from dR, dO, E, S_in and dS_out over all
// value columns: each is written once, with no atomic accumulation.

// L = strict_lower(D o K W^T), M = lower(D o Q W^T) of a chunk's n tokens
// into lm, mm (bf16 operands: the bf16 instruction gives the exact fp32
// sums); D_ji = exp(G_j - G_i)
template <class Sm>
__device__ __forceinline__ void form_lm_bf16(Sm& sm, int n, int wave, int lane) {
  constexpr int PK = Sm::PK, DK = Sm::DKV;
  const int lr = lane & 15, lg = lane >> 4;
  for (int tile = wave; tile < 16; tile += NW) {
    const int tr = tile >> 2, tc = tile & 3;
    f32x4 al = zero4(), am = zero4();
    if (tr >= tc) {
      const uint16_t* kr = sm.k + (16 * tr + lr) * PK;
      const uint16_t* qr = sm.q + (16 * tr + lr) * PK;
      const uint16_t* wr = sm.w + (16 * tc + lr) * PK;
#pragma unroll 4
      for (int k0 = 0; k0 < DK; k0 += 16) {
        const int k_ = k0 + 4 * lg;
        const s16x4 wv = bf4(wr, k_);
        al = mfma16(bf4(kr, k_), wv, al);
        am = mfma16(bf4(qr, k_), wv, am);
      }
    }
    const int i = 16 * tc + lr;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int j = 16 * tr + 4 * lg + ii;
      const float dm = j < n && i <= j ? expf(sm.G[j] - sm.G[i]) : 0.f;
      sm.lm[j * PC + i] = i < j ? dm * al[ii] : 0.f;
      sm.mm[j * PC + i] = dm * am[ii];
    }
  }
}

// k, q, w of chunk c (bf16) and its decay: G, exp(G), exp(G_n - G), and a
// zeroed dL/dG accumulator
template <class Sm>
__device__ __forceinline__ void stage_kqw(Sm& sm, const BwdArgs& a, long tok0, int c, int tid, int lane) {
  constexpr int DK = Sm::DKV, PK = Sm::PK, KV = CH * DK / NT;
  const int t0 = c * CH, n = min(CH, a.T - t0);
  const int kt = tid * KV / DK, kd = tid * KV % DK;
  // every load unconditional (a load under a branch makes the wavefront wait
  // for it where the branches join): rows past the end read the last row
  // and are staged as zeros
  const long krow = (tok0 + t0 + min(kt, n - 1)) * DK + kd;
  const bool kok = kt < n;
  float kv[KV], qv[KV], wv[KV];
  load_vec<uint16_t, KV>(a.k, krow, true, kv);
  load_vec<uint16_t, KV>(a.q, krow, true, qv);
  load_vec<uint16_t, KV>(a.w, krow, true, wv);
  const float alv = static_cast<const float*>(a.g.alpha)[tok0 + t0 + min(lane, n - 1)];
#pragma unroll
  for (int j = 0; j < KV; ++j) {
    sm.k[kt * PK + kd + j] = kok ? f2bf(kv[j]) : 0;
    sm.q[kt * PK + kd + j] = kok ? f2bf(qv[j]) : 0;
    sm.w[kt * PK + kd + j] = kok ? f2bf(wv[j]) : 0;
  }
  if (tid < 64) {
    // inclusive prefix sum of log(alpha) over the chunk (padding: alpha = 1)
    float l = tid < n ? logf(alv) : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(l, off);
      if (lane >= off) l += y;
    }
    sm.G[tid] = l;
    sm.gam[tid] = expf(l);
    sm.fn[tid] = expf(__shfl(l, CH - 1) - l);
    sm.sg[tid] = 0.f;
  }
}

// (I + L_bb)^-1 of the four diagonal 16x16 blocks of I + L, by forward
// substitution (waves 0..3, lane c holds column c)
__device__ __forceinline__ void invert_blocks(const float* lm, float* tb, int wave, int lane) {
  if (wave < 4 && lane < 16) {
    const int b = wave, c = lane;
    float t[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float s = r == c ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < r; ++m) s = fmaf(-lm[(16 * b + r) * PC + 16 * b + m], t[m], s);
      t[r] = s;
      tb[(16 * b + r) * PT + c] = s;
    }
  }
}
// (I + L)^T Z = X in place for ncb 16-column tiles of X (row pitch PX), one
// wave per column tile: Z_b = T_b^T (X_b - sum_{m>b} L_mb^T Z_m), blocks from
// the last; the product's k index runs over the rows a lane holds
template <int PX>
__device__ __forceinline__ void solve_upper(const float* lm, const float* tb, float* X, int ncb, int wave,
                                            int lane) {
  const int lr = lane & 15, lg = lane >> 4;
  for (int cb = wave; cb < ncb; cb += NW)
    for (int b = 3; b >= 0; --b) {
      const f32x4 acc = mm_bf<false, false>(
          zero4(), 16 * (b + 1), CH, [&](int r, int k_) { return lm[k_ * PC + 16 * b + r]; },
          [&](int k_, int cc) { return X[k_ * PX + 16 * cb + cc]; }, lane);
      f32x4 z, u = zero4();
#pragma unroll
      for (int i = 0; i < 4; ++i) z[i] = X[(16 * b + 4 * lg + i) * PX + 16 * cb + lr] - acc[i];
#pragma unroll
      for (int s = 0; s < 4; ++s) u = mfma4(tb[(16 * b + 4 * lg + s) * PT + lr], z[s], u);
#pragma unroll
      for (int i = 0; i < 4; ++i) X[(16 * b + 4 * lg + i) * PX + 16 * cb + lr] = u[i];
      wave_lds_sync();
    }
}

// chunk_bwd_zp_kernel: the dS-independent part of every chunk's
// (I + L)^T dR = M^T dO + W~ dS_out, one workgroup per (b, h, chunk):
// Z = (I + L)^-T W~ [CH, dk] into the workspace as split bf16 pairs (rows past
// the end zero), and P = (I + L)^-T M^T dO [n, dv] into dv_out, in 64-column
// slices.  The serial sweep then needs only dR = P + Z dS_out.
constexpr int PO = 64 + 4;   // row pitch of the 64-column fp32 slices
constexpr int POB = 64 + 8;  // row pitch of the 64-column bf16 dO slice
// At most 80 KiB, so that two workgroups share a compute unit and one's
// memory phases overlap the other's products: k and q take turns in one
// buffer, and W~ / Z, then P and the dO slice, reuse the k / q and w rows
// once L and M are formed.
template <int DK>
struct SmemZ {
  static constexpr int PK = DK + 2;  // bf16 row pitch of the operand rows
  static constexpr int PX = DK + 2;  // fp32 row pitch of x (W~, then Z): the size of kq and w
  static constexpr int XS = CH * PX > CH * PO + CH * POB / 2 ? CH * PX : CH * PO + CH * POB / 2;
  union {
    struct {
      uint16_t kq[CH * PK];  // k, then q
      uint16_t w[CH * PK];
    } r;
    float x[XS];  // W~ solved in place into Z; then P (pitch PO) and dO (bf16, pitch POB)
  } u;
  float lm[CH * PC];  // L
  float mm[CH * PC];  // M
  float tb[4 * 16 * PT];
  float G[CH], fn[CH];
};

template <int DK>
__global__ __launch_bounds__(NT, 2) void chunk_bwd_zp_kernel(BwdArgs a) {
  using Sm = SmemZ<DK>;
  constexpr int PK = Sm::PK, PX = Sm::PX;
  static_assert(sizeof(Sm) <= 80 * 1024, "two workgroups per compute unit");
  static_assert(CH * PO + CH * POB / 2 <= Sm::XS && CH * PX <= Sm::XS, "P and dO in x");
  static_assert(offsetof(Sm, lm) % 16 == 0 && offsetof(Sm, mm) % 16 == 0 && (CH * PO * 4) % 16 == 0,
                "16-byte LDS rows");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  DN_LDS_POISON(smem_raw, sizeof(Sm));
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int T = a.T, dv = a.dv;
  const int nch = (T + CH - 1) / CH;
  const long bh = blockIdx.x / nch;
  const int c = blockIdx.x % nch;
  const int t0 = c * CH, n = min(CH, T - t0);
  const long tok0 = bh * T;
  float* const P = sm.u.x;  // [CH][PO] after Z is out
  uint16_t* const O = reinterpret_cast<uint16_t*>(sm.u.x + CH * PO);  // [CH][POB]

  // k, q, w rows of the chunk (16-byte pieces, rows past the end read the
  // last row and are staged as zeros: no load under a branch), the decay,
  // and the first dO slice, all in one round trip
  constexpr int KP = CH * DK / 8 / NT;  // pieces per thread and array
  static_assert(KP >= 1, "k, q, w pieces");
  u32x4 kr[KP], qr[KP], wr[KP];
  auto piece = [&](int m, int& t, int& d) {
    const int i = tid + NT * m;
    t = i / (DK / 8);
    d = i % (DK / 8) * 8;
  };
#pragma unroll
  for (int m = 0; m < KP; ++m) {
    int t, d;
    piece(m, t, d);
    const long off = (tok0 + t0 + min(t, n - 1)) * DK + d;
    kr[m] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.k) + off);
    qr[m] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + off);
    wr[m] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.w) + off);
  }
  const float alv = static_cast<const float*>(a.g.alpha)[tok0 + t0 + min(lane, n - 1)];
  static_assert(CH * 64 / 8 == NT, "one dO piece per thread");
  const int ot = tid / 8, oc8 = tid % 8 * 8;
  u32x4 od;
  auto fetch_o = [&](int s0) {
    od = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.dO) + (tok0 + t0 + min(ot, n - 1)) * dv +
                                         s0 + oc8);
  };
  fetch_o(0);
  auto put_rows = [&](uint16_t* dst, const u32x4 (&v)[KP]) {
#pragma unroll
    for (int m = 0; m < KP; ++m) {
      int t, d;
      piece(m, t, d);
      // rows at an odd pitch of 2-byte elements: 4-byte stores
      uint32_t* q4 = reinterpret_cast<uint32_t*>(dst + t * PK + d);
#pragma unroll
      for (int j = 0; j < 4; ++j) q4[j] = t < n ? v[m][j] : 0u;
    }
  };
  put_rows(sm.u.r.kq, kr);
  put_rows(sm.u.r.w, wr);
  if (tid < 64) {
    // inclusive prefix sum of log(alpha) over the chunk (padding: alpha = 1)
    float l = tid < n ? logf(alv) : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(l, off);
      if (lane >= off) l += y;
    }
    sm.G[tid] = l;
    sm.fn[tid] = expf(__shfl(l, CH - 1) - l);
  }
  __syncthreads();
  // L = strict_lower(D o K W^T), then M = lower(D o Q W^T), bf16 products
  // (exact in fp32), D_ji = exp(G_j - G_i)
  auto form = [&](float* out, bool strict) {
    for (int tile = wave; tile < 16; tile += NW) {
      const int tr = tile >> 2, tc = tile & 3;
      f32x4 acc = zero4();
      if (tr >= tc) {
        const uint16_t* ar = sm.u.r.kq + (16 * tr + lr) * PK;
        const uint16_t* wr_ = sm.u.r.w + (16 * tc + lr) * PK;
#pragma unroll 4
        for (int k0 = 0; k0 < DK; k0 += 16) acc = mfma16(bf4(ar, k0 + 4 * lg), bf4(wr_, k0 + 4 * lg), acc);
      }
      const int i = 16 * tc + lr;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int j = 16 * tr + 4 * lg + ii;
        const float dm = j < n && i <= j ? expf(sm.G[j] - sm.G[i]) : 0.f;
        out[j * PC + i] = !strict || i < j ? dm * acc[ii] : 0.f;
      }
    }
  };
  form(sm.lm, true);
  __syncthreads();
  put_rows(sm.u.r.kq, qr);
  __syncthreads();
  form(sm.mm, false);
  // W~ = diag(g_n / g) W into registers (rows past the end zero: w staged as
  // 0), then into x once every reader of the rows is done
  constexpr int XV = CH * DK / NT;
  float wt[XV];
#pragma unroll
  for (int j = 0; j < XV; ++j) {
    const int idx = tid * XV + j, t = idx / DK, d = idx % DK;
    wt[j] = sm.fn[t] * bf2f(sm.u.r.w[t * PK + d]);
  }
  __syncthreads();
  invert_blocks(sm.lm, sm.tb, wave, lane);
#pragma unroll
  for (int j = 0; j < XV; ++j) {
    const int idx = tid * XV + j, t = idx / DK, d = idx % DK;
    sm.u.x[t * PX + d] = wt[j];
  }
  __syncthreads();
  solve_upper<PX>(sm.lm, sm.tb, sm.u.x, DK / 16, wave, lane);
  __syncthreads();
  {
    u32x4* zo = reinterpret_cast<u32x4*>(a.Z_ck + (bh * nch + c) * CH * DK);
    for (int idx = tid; idx < CH * DK / 4; idx += NT) {
      const int t = idx / (DK / 4), d = idx % (DK / 4) * 4;
      const float* xr = sm.u.x + t * PX + d;
      zo[idx] = u32x4{split_bf(xr[0]), split_bf(xr[1]), split_bf(xr[2]), split_bf(xr[3])};
    }
  }
  for (int s0 = 0; s0 < dv; s0 += 64) {
    __syncthreads();  // the previous readers of x (Z, then P) are done
    *reinterpret_cast<u32x4*>(O + ot * POB + oc8) = ot < n ? od : u32x4{0u, 0u, 0u, 0u};
    // the next slice (at the last, a harmless repeat of it)
    fetch_o(min(s0 + 64, dv - 64));
    __syncthreads();
    // M^T dO (rows past the end zero)
    for (int tile = wave; tile < 16; tile += NW) {
      const int ib = tile >> 2, cb = tile & 3;
      const f32x4 acc = mm_bf<false, true>(
          zero4(), 16 * ib, CH, [&](int r, int k_) { return sm.mm[k_ * PC + 16 * ib + r]; },
          [&](int k_, int cc) { return bf2f(O[k_ * POB + 16 * cb + cc]); }, lane);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) P[(16 * ib + 4 * lg + ii) * PO + 16 * cb + lr] = acc[ii];
    }
    __syncthreads();
    solve_upper<PO>(sm.lm, sm.tb, P, 4, wave, lane);
    __syncthreads();
    {
      const int t = tid / 8, c8 = tid % 8 * 8;
      if (t < n) {
        f32x4* dst = reinterpret_cast<f32x4*>(a.dv_out + (tok0 + t0 + t) * dv + s0 + c8);
        const float* xr = P + t * PO + c8;
        dst[0] = f32x4{xr[0], xr[1], xr[2], xr[3]};
        dst[1] = f32x4{xr[4], xr[5], xr[6], xr[7]};
      }
    }
  }
}

// chunk_bwd_ds_kernel: the serial sweep, one workgroup of four wavefronts per
// (b, h, 64 value columns); wavefront j owns value columns 16 j .. 16 j + 15
// of the slice and holds that d_k x 16 slice of dS in registers, in the
// accumulator layout of a 16x16 tile per 16 key channels.  From the last
// chunk, per chunk: dR = P + Z dS_out (written to dv_out, where the tile
// kernel reads it as dR), dS_out stored for the tile kernel, then
// dS_in = g_n dS_out + Q^T (g dO) - K^T (g dR).  Z, k, q and the decay of the
// next chunk are loaded while the current chunk runs and staged into the
// other half of a double buffer after it; P and dO are loaded into registers
// a step ahead.  Every global access is issued unconditionally: loads and
// stores of a partial chunk go through buffer resources sized to its n
// tokens, so rows past the end read as zero and their stores are dropped
// (a load under a branch makes the wavefront wait for it where the branches
// join).  Products run on v_mfma_f32_16x16x32_bf16: Z and dS as split pairs
// (three instructions), q and k exact against the split fp32 side (two).
// The 32 k-slots of one instruction are taken as rows 4 g + i (i < 4) of the
// first 16-block and 4 g + i - 4 of the second (g = lane / 16), in both
// operands.
constexpr int NTS = 256;  // threads of the serial sweep
constexpr int DVS_S = 64; // value columns per workgroup of the serial sweep
typedef short s16x4_lds __attribute__((ext_vector_type(4), address_space(3)));
// rows r0 + 4 g + j (j < 4), column c0 + lane % 16 of a row-major bf16 array
// of pitch ld in LDS, in one ds_read_b64_tr_b16 (within each group of 16
// lanes, lane l receives element l % 4 of the 8-byte piece addressed by lane
// 4 j + l / 4)
__device__ __forceinline__ s16x4 read_tr(const uint16_t* p, int ld, int lane, int r0, int c0) {
  const uint16_t* q = p + (r0 + 4 * (lane >> 4) + ((lane & 15) >> 2)) * ld + c0 + 4 * (lane & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_lds*)(q));
}
__device__ __forceinline__ bf16x8 cat8(s16x4 lo, s16x4 hi) {
  const u32x2 x = __builtin_bit_cast(u32x2, lo), y = __builtin_bit_cast(u32x2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{x[0], x[1], y[0], y[1]});
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ s16x4 hi4v(f32x4 v) {
  const float x[4] = {v[0], v[1], v[2], v[3]};
  return hi4(x);
}
__device__ __forceinline__ s16x4 lo4v(f32x4 v) {
  const float x[4] = {v[0], v[1], v[2], v[3]};
  return lo4(x);
}
// a buffer resource over nbytes from base: loads beyond read as zero,
// stores beyond are dropped
__device__ __forceinline__ __amdgpu_buffer_rsrc_t brsrc(const void* base, long nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(nbytes), 0x00020000);
}

template <int DK>
struct SmemS {
  static constexpr int PZ = DK + 4;   // u32 row pitch of Z: rows 16 banks apart per four
  static constexpr int PK = DK + 16;  // bf16 row pitch of k and q (transposing reads)
  uint32_t z[2][CH * PZ];
  uint16_t k[2][CH * PK], q[2][CH * PK];
  float gam[2][CH];  // exp(G_t)
};

template <int DK, bool SUMMARY>
__global__ __launch_bounds__(NTS) void chunk_bwd_ds_kernel(BwdArgs a) {
  using Sm = SmemS<DK>;
  constexpr int PZ = Sm::PZ, PK = Sm::PK, ND = DK / 16, NS = DK / 32;
  constexpr int ZV = CH * DK / 4 / NTS, KV = CH * DK / 8 / NTS;  // 16-byte pieces per thread
  static_assert(ZV >= 1 && KV >= 1 && DVS_S == 16 * (NTS / 64), "serial sweep shape");
  static_assert(offsetof(Sm, z) % 16 == 0 && offsetof(Sm, k) % 16 == 0 && offsetof(Sm, q) % 16 == 0 &&
                    offsetof(Sm, gam) % 16 == 0 && (CH * PZ * 4) % 16 == 0 && (CH * PK * 2) % 16 == 0,
                "16-byte LDS rows");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  DN_LDS_POISON(smem_raw, sizeof(Sm));
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4;
  const int T = a.T, dv = a.dv;
  const int nch = (T + CH - 1) / CH;
  // Segments: chunks [seg nch / nseg, (seg + 1) nch / nseg) of a head (nseg =
  // 1: the whole sequence).  SUMMARY: from dS_out = 0 over the value slices
  // (B of the segment's affine map dS_in = A dS_out + B) and from the
  // identity over DK more columns with dO = P = 0 (A), written to segB and
  // segA under the index nseg - 1 - seg (the order segment_combine_kernel
  // chains them in, from dS_T).  Otherwise from dS_T (nseg = 1) or from the
  // chained dS_out of the segment (seg_in), storing dS_out and dR per chunk.
  const int nseg = a.nseg;
  const int nslv = dv / DVS_S;
  const int nsl = SUMMARY ? nslv + DK / DVS_S : nslv;
  // the slices of one head and segment on one XCD (consecutive workgroup ids
  // go to the 8 XCDs in turn), so that they share its L2 copy of Z, k and q
  const unsigned G = gridDim.x;
  const unsigned lin = G % 8 == 0 ? (blockIdx.x % 8) * (G / 8) + blockIdx.x / 8 : blockIdx.x;
  const long hs = lin / nsl;
  const int sl = static_cast<int>(lin % nsl);
  const long bh = hs / nseg;
  const int seg = static_cast<int>(hs % nseg);
  const int rs = nseg - 1 - seg;
  const bool tmap = SUMMARY && sl >= nslv;  // identity columns: the transfer map A
  // this lane's value column (identity column of A on a tmap slice)
  const int col = (tmap ? sl - nslv : sl) * DVS_S + 16 * wave + (lane & 15);
  const int c_lo = static_cast<int>(static_cast<long>(seg) * nch / nseg);
  const int c_hi = static_cast<int>(static_cast<long>(seg + 1) * nch / nseg);
  const long tok0 = bh * T;
  const uint16_t* kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* og = static_cast<const uint16_t*>(a.dO);
  const float* alg = static_cast<const float*>(a.g.alpha);
  auto nof = [&](int c) { return min(CH, T - c * CH); };
  // this lane's rows 4 g + i of a [CH][dv] array: byte offset of row 4 g and
  // column col; the rows 16 ib + i are scalar offsets
  const int loff = (4 * lg * dv + col);

  u32x4 zr[ZV], kr[KV], qr[KV];
  float al;
  float pn[4][4];     // P of this lane's rows
  uint16_t on[4][4];  // dO of this lane's rows, bf16
  // Z, k, q and alpha of chunk c, issued at the start of a step and used when
  // it ends; the decay first, so that waiting for the group waits for nothing
  // issued later
  auto fetch_a = [&](int c) {
    const int t0 = c * CH, n = nof(c);
    al = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(brsrc(alg + tok0 + t0, 4 * n), 4 * lane, 0, 0));
    const u32x4* zs = reinterpret_cast<const u32x4*>(a.Z_ck + (bh * nch + c) * CH * DK);
#pragma unroll
    for (int m = 0; m < ZV; ++m) zr[m] = zs[tid + NTS * m];
    const auto rk = brsrc(kg + (tok0 + t0) * DK, 2l * n * DK), rq = brsrc(qg + (tok0 + t0) * DK, 2l * n * DK);
#pragma unroll
    for (int m = 0; m < KV; ++m) {
      kr[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, 16 * tid, 16 * NTS * m, 0));
      qr[m] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, 16 * tid, 16 * NTS * m, 0));
    }
  };
  // P and dO of chunk c, issued just before a step ends and used halfway
  // through the next
  auto fetch_b = [&](int c) {
    const int t0 = c * CH, n = nof(c);
    // (no P or dO on the identity columns: empty resources, loads read zero)
    const auto rp = brsrc(a.dv_out + (tok0 + t0) * dv, tmap ? 0 : 4l * n * dv);
    const auto ro = brsrc(og + (tok0 + t0) * dv, tmap ? 0 : 2l * n * dv);
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int so = (16 * ib + i) * dv;
        pn[ib][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rp, 4 * loff, 4 * so, 0));
        on[ib][i] = __builtin_amdgcn_raw_buffer_load_b16(ro, 2 * loff, 2 * so, 0);
      }
  };
  // stage the fetched chunk (n tokens) into half b of the double buffer
  auto put = [&](int b, int n) {
#pragma unroll
    for (int m = 0; m < ZV; ++m) {
      const int idx = tid + NTS * m, t = idx / (DK / 4), d = idx % (DK / 4) * 4;
      *reinterpret_cast<u32x4*>(&sm.z[b][t * PZ + d]) = zr[m];
    }
#pragma unroll
    for (int m = 0; m < KV; ++m) {
      const int idx = tid + NTS * m, t = idx / (DK / 8), d = idx % (DK / 8) * 8;
      *reinterpret_cast<u32x4*>(&sm.k[b][t * PK + d]) = kr[m];
      *reinterpret_cast<u32x4*>(&sm.q[b][t * PK + d]) = qr[m];
    }
    if (wave == 0) {
      // inclusive prefix sum of log(alpha) over the chunk (padding: alpha = 1)
      float l = lane < n ? logf(al) : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(l, off);
        if (lane >= off) l += y;
      }
      sm.gam[b][lane] = expf(l);
    }
  };

  f32x4 dS[ND];
  {
    // the entering dS_out: dS_T or seg_in (none: an empty resource, every
    // load reads zero; SUMMARY: zero, or the identity on the tmap slices)
    const float* src = SUMMARY ? nullptr : nseg > 1 ? a.seg_in + (bh * nseg + rs) * DK * dv
                                                    : a.dS_T ? a.dS_T + bh * DK * dv : nullptr;
    const auto rt = brsrc(src, src ? 4l * DK * dv : 0);
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rt, 4 * loff, 4 * (16 * db + i) * dv, 0));
        dS[db][i] = tmap ? (16 * db + 4 * lg + i == col ? 1.f : 0.f) : x;
      }
  }
  fetch_a(c_hi - 1);
  put((c_hi - 1) & 1, nof(c_hi - 1));
  fetch_b(c_hi - 1);
  __syncthreads();
  for (int c = c_hi - 1; c >= c_lo; --c) {
    const int b = c & 1, t0 = c * CH, n = nof(c);
    // the next chunk's loads (at the segment's first chunk, harmless repeats
    // of it: every step issues the same loads, so no wait depends on the path)
    const int cn = max(c - 1, c_lo);
    fetch_a(cn);
    // keep the scheduler from sinking these loads towards their use
    __builtin_amdgcn_sched_barrier(0);
    // dS_out^T [dv][dk] of the chunk for the tile kernel: each lane's four key
    // channels are one 16-byte piece
    if constexpr (!SUMMARY) {
      f32x4* dsk = reinterpret_cast<f32x4*>(a.dS_ck + ((bh * nch + c) * dv + col) * DK + 4 * lg);
#pragma unroll
      for (int db = 0; db < ND; ++db) dsk[4 * db] = dS[db];
    }
    // dS_out as split pairs
    bf16x8 sh[NS], sl[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      sh[s] = cat8(hi4v(dS[2 * s]), hi4v(dS[2 * s + 1]));
      sl[s] = cat8(lo4v(dS[2 * s]), lo4v(dS[2 * s + 1]));
    }
    // Y = Z dS_out; dR = P + Y (to dv_out); the g-scaled split operands of
    // the dS_in products
    const uint32_t* zb = sm.z[b];
    const auto rdr = brsrc(a.dv_out + (tok0 + t0) * dv, 4l * n * dv);
    f32x4 yt[4];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      f32x4 y = zero4();
      const uint32_t* zrow = zb + (16 * ib + (lane & 15)) * PZ + 4 * lg;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 z0 = *reinterpret_cast<const u32x4*>(zrow + 32 * s);
        const u32x4 z1 = *reinterpret_cast<const u32x4*>(zrow + 32 * s + 16);
        s16x4 h0, l0, h1, l1;
        split4(z0[0], z0[1], z0[2], z0[3], h0, l0);
        split4(z1[0], z1[1], z1[2], z1[3], h1, l1);
        const bf16x8 zh = cat8(h0, h1), zl = cat8(l0, l1);
        y = mfma32(zh, sh[s], mfma32(zh, sl[s], mfma32(zl, sh[s], y)));
      }
      yt[ib] = y;
    }
    // P and dO are used only from here
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 oh[2], ol[2], rh[2], rl[2];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
      const f32x4 y = yt[ib];
      const f32x4 g4 = *reinterpret_cast<const f32x4*>(&sm.gam[b][16 * ib + 4 * lg]);
      f32x4 go, gr;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // rows past the end: P and dO read as zero, Z's rows are zero
        const float dr = pn[ib][i] + y[i];
        if constexpr (!SUMMARY)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dr), rdr, 4 * loff, 4 * (16 * ib + i) * dv, 0);
        go[i] = g4[i] * bf2f(on[ib][i]);
        gr[i] = -g4[i] * dr;
      }
      // tile ib is half ib % 2 of the 32-token operand ib / 2
      const s16x4 goh = hi4v(go), gol = lo4v(go), grh = hi4v(gr), grl = lo4v(gr);
      if (ib % 2 == 0) {
        oh[ib / 2] = cat8(goh, goh);
        ol[ib / 2] = cat8(gol, gol);
        rh[ib / 2] = cat8(grh, grh);
        rl[ib / 2] = cat8(grl, grl);
      } else {
        auto sethi = [](bf16x8& v, s16x4 h) {
          const u32x2 x = __builtin_bit_cast(u32x2, h);
          u32x4 u = __builtin_bit_cast(u32x4, v);
          u[2] = x[0], u[3] = x[1];
          v = __builtin_bit_cast(bf16x8, u);
        };
        sethi(oh[ib / 2], goh);
        sethi(ol[ib / 2], gol);
        sethi(rh[ib / 2], grh);
        sethi(rl[ib / 2], grl);
      }
    }
    // dS_in = g_n dS_out + Q^T (g dO) - K^T (g dR)
    const float gn = sm.gam[b][CH - 1];
    const uint16_t *qb = sm.q[b], *kb = sm.k[b];
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      f32x4 acc = gn * dS[db];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 qa = cat8(read_tr(qb, PK, lane, 32 * s, 16 * db), read_tr(qb, PK, lane, 32 * s + 16, 16 * db));
        const bf16x8 ka = cat8(read_tr(kb, PK, lane, 32 * s, 16 * db), read_tr(kb, PK, lane, 32 * s + 16, 16 * db));
        acc = mfma32(qa, oh[s], mfma32(qa, ol[s], acc));
        acc = mfma32(ka, rh[s], mfma32(ka, rl[s], acc));
      }
      dS[db] = acc;
    }
    __builtin_amdgcn_sched_barrier(0);
    fetch_b(cn);
    __builtin_amdgcn_sched_barrier(0);
    put(b ^ 1, nof(cn));
    __syncthreads();
  }
  if constexpr (SUMMARY) {
    // A [DK][DK] (row d, identity column col) or B [DK][dv] of the segment
    float* dst = tmap ? a.segA + (bh * nseg + rs) * DK * DK : a.segB + (bh * nseg + rs) * DK * dv;
    const int ld = tmap ? DK : dv;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) dst[(16 * db + 4 * lg + i) * ld + col] = dS[db][i];
  } else if (nseg == 1 && a.dS0) {
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.dS0[(bh * DK + 16 * db + 4 * lg + i) * dv + col] = dS[db][i];
  }
}

template <int DK>
struct SmemT {
  static constexpr int DKV = DK;
  static constexpr int VS = 32;      // value columns per slice of the contractions
  static constexpr int PH = VS + 8;  // bf16 row pitch of the split planes (16-byte pieces)
  static constexpr int PK = DK + 16; // bf16 row pitch of k, q, w (transposing reads)
  uint16_t k[CH * PK], q[CH * PK], w[CH * PK];
  // one value slice as bf16 planes: hi = bf16(v), lo = bf16(v - hi)
  uint16_t Sh[DK * PH], Sl[DK * PH], dSh[DK * PH], dSl[DK * PH];  // S_in, dS_out [key][col]
  uint16_t eh[CH * PH], el[CH * PH], yh[CH * PH], yl[CH * PH];    // E, dR [token][col]
  uint16_t xh[CH * PH];                                           // dO (bf16)
  float lm[CH * PC];  // L, then D o dL as split words
  float mm[CH * PC];  // M, then D o dM as split words
  float G[CH], gam[CH], fn[CH], sg[CH];
};

template <int DK, int FUSE>
__global__ __launch_bounds__(NT) void chunk_bwd_tiles_kernel(BwdArgs a) {
  using Sm = SmemT<DK>;
  constexpr int PK = Sm::PK, VS = Sm::VS, PH = Sm::PH;
  constexpr int ND = DK / 16;
  constexpr int TPW = 4 * ND / NW;  // [token][key] tiles per wavefront
  static_assert(TPW * NW == 4 * ND, "key tiles per wavefront");
  static_assert(offsetof(Sm, Sh) % 16 == 0 && offsetof(Sm, Sl) % 16 == 0 && offsetof(Sm, dSh) % 16 == 0 &&
                    offsetof(Sm, dSl) % 16 == 0 && offsetof(Sm, eh) % 16 == 0 && offsetof(Sm, el) % 16 == 0 &&
                    offsetof(Sm, yh) % 16 == 0 && offsetof(Sm, yl) % 16 == 0 && offsetof(Sm, xh) % 16 == 0 &&
                    offsetof(Sm, lm) % 16 == 0 && offsetof(Sm, mm) % 16 == 0 && (PH * 2) % 16 == 0 &&
                    (PK * 2) % 8 == 0,
                "16-byte LDS rows");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  DN_LDS_POISON(smem_raw, sizeof(Sm));
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int T = a.T, dv = a.dv;
  const int nch = (T + CH - 1) / CH;
  const long bh = blockIdx.x / nch;
  const int c = blockIdx.x % nch;
  const int t0 = c * CH, n = min(CH, T - t0);
  const long tok0 = bh * T;
  auto kf = [&](int t, int d) { return bf2f(sm.k[t * PK + d]); };
  auto qf = [&](int t, int d) { return bf2f(sm.q[t * PK + d]); };
  auto wf = [&](int t, int d) { return bf2f(sm.w[t * PK + d]); };

  // the value slices' operands, each fetched into registers one slice ahead
  // (the first while L and M are formed): S_in rows sd, columns sc..; dS_out
  // (stored transposed, [dv][dk] per chunk) SV key channels from tdk of
  // column tcol; E, dR (= dV) and dO of token xt, columns xc..  Rows past the end
  // read the last row and are stored as zeros (no load under a branch).
  constexpr int SV = DK * VS / NT, XV = CH * VS / NT;
  const int sd = tid * SV / VS, sc = tid * SV % VS;
  const int xt = tid * XV / VS, xc = tid * XV % VS;
  const int tcol = tid * SV / DK, tdk = tid * SV % DK;
  const bool xok = xt < n;
  const int nsl = dv / VS;
  float pS[SV], pdS[SV], pE[XV], pR[XV], pO[XV];
  auto fetch_slice = [&](int s) {
    const int col0 = s * VS;
    const long srow = ((bh * nch + c) * DK + sd) * dv + col0 + sc;
    const long trow = ((bh * nch + c) * dv + col0 + tcol) * DK + tdk;
    const long xrow = (tok0 + t0 + min(xt, n - 1)) * dv + col0 + xc;
    load_vec<float, SV>(a.S_ck, srow, true, pS);
    load_vec<float, SV>(a.dS_ck, trow, true, pdS);
    load_vec<float, XV>(a.E, xrow, true, pE);
    load_vec<float, XV>(a.dv_out, xrow, true, pR);  // dR = dV
    load_vec<uint16_t, XV>(a.dO, xrow, true, pO);
  };

  stage_kqw(sm, a, tok0, c, tid, lane);
  __syncthreads();
  fetch_slice(0);
  form_lm_bf16(sm, n, wave, lane);  // L, M (for the decay's gradient)

  // the contractions over the value columns, 32 at a time: dL = -dR E^T,
  // dM = dO E^T (this wave's lower tiles of the 16: wave and wave + 8), and
  // per (token, key) tile dR S_in^T, dO S_in^T, E dS_out^T; and <S_in, dS_out>
  f32x4 al[2] = {zero4(), zero4()}, am[2] = {zero4(), zero4()};
  f32x4 akh[TPW], aqh[TPW], atw[TPW];
#pragma unroll
  for (int k = 0; k < TPW; ++k) akh[k] = aqh[k] = atw[k] = zero4();
  float sdot = 0.f;
  // the split planes of one value: hi = bf16(v) (RNE), lo = bf16(v - hi)
  auto hl = [](float v, uint16_t& h, uint16_t& l) {
    h = f2bf(v);
    l = f2bf(v - bf2f(h));
  };
  // 8 consecutive k (value columns 8 g .. 8 g + 7 of the slice) of a plane's
  // row, as one v_mfma_f32_16x16x32_bf16 operand
  auto frag = [&](const uint16_t* plane, int row) {
    return *reinterpret_cast<const bf16x8*>(plane + row * PH + 8 * lg);
  };
  for (int s = 0; s < nsl; ++s) {
    __syncthreads();  // the previous slice's readers are done
    {
      static_assert((SV == 8 || SV == 4) && XV == 4, "staging pieces");
      uint16_t h[SV], l[SV];
#pragma unroll
      for (int j = 0; j < SV; ++j) hl(pS[j], h[j], l[j]);
      auto stS = [&](uint16_t* plane, const uint16_t (&v)[SV]) {
        if constexpr (SV == 8)
          *reinterpret_cast<u32x4*>(&plane[sd * PH + sc]) =
              u32x4{pack16(v[0], v[1]), pack16(v[2], v[3]), pack16(v[4], v[5]), pack16(v[6], v[7])};
        else
          *reinterpret_cast<u32x2*>(&plane[sd * PH + sc]) = u32x2{pack16(v[0], v[1]), pack16(v[2], v[3])};
      };
      stS(sm.Sh, h);
      stS(sm.Sl, l);
#pragma unroll
      for (int j = 0; j < SV; ++j) {
        uint16_t hh, ll;
        hl(pdS[j], hh, ll);
        sm.dSh[(tdk + j) * PH + tcol] = hh;
        sm.dSl[(tdk + j) * PH + tcol] = ll;
      }
      uint16_t eh4[XV], el4[XV], yh4[XV], yl4[XV], xh4[XV];
#pragma unroll
      for (int j = 0; j < XV; ++j) {
        hl(xok ? pE[j] : 0.f, eh4[j], el4[j]);
        hl(xok ? pR[j] : 0.f, yh4[j], yl4[j]);
        xh4[j] = xok ? f2bf(pO[j]) : 0;  // dO is a bf16 number
      }
      auto st4 = [&](uint16_t* plane, const uint16_t (&v)[XV]) {
        *reinterpret_cast<u32x2*>(&plane[xt * PH + xc]) = u32x2{pack16(v[0], v[1]), pack16(v[2], v[3])};
      };
      st4(sm.eh, eh4);
      st4(sm.el, el4);
      st4(sm.yh, yh4);
      st4(sm.yl, yl4);
      st4(sm.xh, xh4);
    }
    // the next slice (at the last, a harmless repeat of it)
    fetch_slice(min(s + 1, nsl - 1));
    __syncthreads();
    {
      // <S_in, dS_out> over this thread's piece of the slice (hi + lo within
      // 2^-17 of each value)
#pragma unroll
      for (int j = 0; j < SV; ++j) {
        const int o = sd * PH + sc + j;
        sdot = fmaf(bf2f(sm.Sh[o]) + bf2f(sm.Sl[o]), bf2f(sm.dSh[o]) + bf2f(sm.dSl[o]), sdot);
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int tile = wave + 8 * k, tr = tile >> 2, tc = tile & 3;
      if (tr < tc) continue;  // uniform
      const bf16x8 eh = frag(sm.eh, 16 * tc + lr), el = frag(sm.el, 16 * tc + lr);
      const bf16x8 yh = frag(sm.yh, 16 * tr + lr), yl = frag(sm.yl, 16 * tr + lr), xh = frag(sm.xh, 16 * tr + lr);
      al[k] = mfma32(yh, eh, mfma32(yh, el, mfma32(yl, eh, al[k])));
      am[k] = mfma32(xh, eh, mfma32(xh, el, am[k]));
    }
#pragma unroll
    for (int k = 0; k < TPW; ++k) {
      const int tile = wave + NW * k, tb_ = tile / ND, db = tile % ND;
      const bf16x8 sh = frag(sm.Sh, 16 * db + lr), sl = frag(sm.Sl, 16 * db + lr);
      const bf16x8 dh = frag(sm.dSh, 16 * db + lr), dl = frag(sm.dSl, 16 * db + lr);
      const bf16x8 yh = frag(sm.yh, 16 * tb_ + lr), yl = frag(sm.yl, 16 * tb_ + lr);
      const bf16x8 xh = frag(sm.xh, 16 * tb_ + lr);
      const bf16x8 eh = frag(sm.eh, 16 * tb_ + lr), el = frag(sm.el, 16 * tb_ + lr);
      akh[k] = mfma32(yh, sh, mfma32(yh, sl, mfma32(yl, sh, akh[k])));
      aqh[k] = mfma32(xh, sh, mfma32(xh, sl, aqh[k]));
      atw[k] = mfma32(eh, dh, mfma32(eh, dl, mfma32(el, dh, atw[k])));
    }
  }
  // dL/dG of the chunk end: g_n <S_in, dS_out>
  sdot = wave_total(sdot);
  if (lane == 0) atomicAdd(&sm.sg[CH - 1], sm.gam[CH - 1] * sdot);
  // the decay terms of L and M (L o dL, M o dM: + to the row token, - to the
  // column token), then D o dL and D o dM as split words (entries not
  // written stay 0)
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int tile = wave + 8 * k, tr = tile >> 2, tc = tile & 3;
    if (tr < tc) continue;  // uniform
    const int i = 16 * tc + lr;
    float col = 0.f;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int j = 16 * tr + 4 * lg + ii;
      const bool ok = j < n && i <= j;
      const float dl = -al[k][ii], dmv = am[k][ii];
      float tlm = 0.f;
      if (ok) {
        const float dm = expf(sm.G[j] - sm.G[i]);
        tlm = (i < j ? sm.lm[j * PC + i] * dl : 0.f) + sm.mm[j * PC + i] * dmv;
        if (i == j) tlm = 0.f;  // the diagonal adds and subtracts the same term
        reinterpret_cast<uint32_t*>(sm.lm)[j * PC + i] = split_bf(i < j ? dm * dl : 0.f);
        reinterpret_cast<uint32_t*>(sm.mm)[j * PC + i] = split_bf(dm * dmv);
      }
      col -= tlm;
      const float row = row16_sum(tlm);
      if (lr == 0 && j < n) atomicAdd(&sm.sg[j], row);
    }
    col = col4_sum(col);
    if (lg == 0) atomicAdd(&sm.sg[i], col);
  }
  __syncthreads();
  // per (token, key channel): dk = g (-S_in dR) + (D o dL) W, dq = g S_in dO +
  // (D o dM) W, dw = (g_n / g) dS_out E + (D o dL)^T K + (D o dM)^T Q, and
  // their decay terms
  const uint32_t* lmu = reinterpret_cast<const uint32_t*>(sm.lm);
  const uint32_t* mmu = reinterpret_cast<const uint32_t*>(sm.mm);
  float wend = 0.f;  // the chunk end's part of the W~ terms
  // FUSE (KLA, GDN): the state part of dk and dw per (token, key channel) go
  // to LDS, over the value-slice planes (no longer read), for the write
  // gain's backward below; otherwise dk and dw_acc go to memory
  constexpr int PSC = DK + 1;
  static_assert(2 * CH * PSC * 4 <= offsetof(Sm, lm) - offsetof(Sm, Sh), "dk / dw scratch");
  float* const scr_dk = reinterpret_cast<float*>(sm.Sh);
  float* const scr_dw = scr_dk + CH * PSC;
#pragma unroll
  for (int k = 0; k < TPW; ++k) {  // unrolled: the accumulators stay in registers
    const int tile = wave + NW * k, tb_ = tile / ND, db = tile % ND;
    f32x4 ask = zero4(), asq = zero4(), asw = zero4(), asw2 = zero4();
#pragma unroll 2
    for (int k0 = 0; k0 < 16 * (tb_ + 1); k0 += 16) {
      const int k_ = k0 + 4 * lg;
      const s16x4 wv = read_tr(sm.w, PK, lane, k0, 16 * db);
      const u32x4 lw = *reinterpret_cast<const u32x4*>(lmu + (16 * tb_ + lr) * PC + k_);
      const u32x4 mw = *reinterpret_cast<const u32x4*>(mmu + (16 * tb_ + lr) * PC + k_);
      s16x4 h, l;
      split4(lw[0], lw[1], lw[2], lw[3], h, l);
      ask = mfma16(l, wv, mfma16(h, wv, ask));
      split4(mw[0], mw[1], mw[2], mw[3], h, l);
      asq = mfma16(l, wv, mfma16(h, wv, asq));
    }
#pragma unroll 2
    for (int k0 = 16 * tb_; k0 < CH; k0 += 16) {
      const int k_ = k0 + 4 * lg;
      const uint32_t* lc = lmu + k_ * PC + 16 * tb_ + lr;
      const uint32_t* mc = mmu + k_ * PC + 16 * tb_ + lr;
      s16x4 h, l;
      split4(lc[0], lc[PC], lc[2 * PC], lc[3 * PC], h, l);
      const s16x4 kv = read_tr(sm.k, PK, lane, k0, 16 * db);
      asw = mfma16(l, kv, mfma16(h, kv, asw));
      split4(mc[0], mc[PC], mc[2 * PC], mc[3 * PC], h, l);
      const s16x4 qv = read_tr(sm.q, PK, lane, k0, 16 * db);
      asw2 = mfma16(l, qv, mfma16(h, qv, asw2));
    }
    asw += asw2;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int t = 16 * tb_ + 4 * lg + ii, d = 16 * db + lr;
      const bool ok = t < n;
      const long gi = (tok0 + t0 + t) * DK + d;
      const float kh = -akh[k][ii], qh = aqh[k][ii], tw = atw[k][ii];
      const float kv = kf(t, d), qv = qf(t, d), wv = wf(t, d);
      const float g = sm.gam[t], f = sm.fn[t];
      const float wtw = f * wv * tw;
      if (ok) {
        a.dq_out[gi] = fmaf(g, qh, asq[ii]);
        if constexpr (FUSE != FUSE_NONE) {
          scr_dk[t * PSC + d] = fmaf(g, kh, ask[ii]);
          scr_dw[t * PSC + d] = fmaf(f, tw, asw[ii]);
        } else {
          a.dk_out[gi] = fmaf(g, kh, ask[ii]);
          a.dw_acc[gi] = fmaf(f, tw, asw[ii]);
        }
        wend += wtw;
      }
      const float row = row16_sum(ok ? g * (kv * kh + qv * qh) - wtw : 0.f);
      if (lr == 0 && ok) atomicAdd(&sm.sg[t], row);
    }
  }
  wend = wave_total(wend);
  if (lane == 0) atomicAdd(&sm.sg[CH - 1], wend);
  __syncthreads();
  if constexpr (FUSE != FUSE_NONE) {
    // the write gain's backward (as gain_bwd_tok_kernel): DK / 16 threads
    // per token, 16 key channels each; k . dw and ||k||^2 summed over those
    // lanes.  KLA: w = beta k, beta = eta / (||k||^2 + eps); GDN: w = eta k.
    // (DK 64: threads past the chunk's 64 tokens read its last row, write
    // nothing)
    constexpr int TPT = DK / 16;
    static_assert(NT / TPT >= CH, "a thread group per token");
    const int t = tid / TPT, d0 = tid % TPT * 16, tr = min(t, CH - 1);
    float dkv[16], dwv[16], kv[16];
    float db = 0.f, n2 = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      kv[j] = kf(tr, d0 + j);
      dkv[j] = scr_dk[tr * PSC + d0 + j];
      dwv[j] = scr_dw[tr * PSC + d0 + j];
      db = fmaf(dwv[j], kv[j], db);
      n2 = fmaf(kv[j], kv[j], n2);
    }
#pragma unroll
    for (int m = 1; m < TPT; m <<= 1) {
      db += __shfl_xor(db, m);
      n2 += __shfl_xor(n2, m);
    }
    if (t < n) {
      const long ti = tok0 + t0 + t;
      const float et = a.g.eta[ti];
      float deta;
      if constexpr (FUSE == FUSE_KLA) {
        const float den = n2 + a.g.eps, beta = et / den, g2 = db * (-et / (den * den));
#pragma unroll
        for (int j = 0; j < 16; ++j) dkv[j] = fmaf(beta, dwv[j], fmaf(2.f * kv[j], g2, dkv[j]));
        deta = db / den;
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) dkv[j] = fmaf(et, dwv[j], dkv[j]);
        deta = db;
      }
      f32x4* dst = reinterpret_cast<f32x4*>(a.dk_out + ti * DK + d0);
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[j] = f32x4{dkv[4 * j], dkv[4 * j + 1], dkv[4 * j + 2], dkv[4 * j + 3]};
      if (d0 == 0) a.deta[ti] = deta;
    }
    // dL/dalpha_t = (sum of dL/dG_j over the chunk's j >= t) / alpha_t: lane
    // l of wavefront 0 takes token n - 1 - l, so that its prefix sum over the
    // lanes is the suffix sum over the tokens; the padding tokens of a
    // partial chunk share the last real token's decay
    if (tid < CH) {
      const int tt = n - 1 - tid;
      float tail = 0.f;
      if (tid == 0)
        for (int u = n; u < CH; ++u) tail += sm.sg[u];
      float sfx = tt >= 0 ? sm.sg[tt] + tail : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(sfx, off);
        if (lane >= off) sfx += y;
      }
      if (tt >= 0)
        a.dalpha[tok0 + t0 + tt] = sfx / static_cast<const float*>(a.g.alpha)[tok0 + t0 + tt];
    }
  } else if (tid < CH) {
    // dL/dG of the chunk's tokens; the padding tokens of a partial chunk share
    // the last real token's decay
    const float v = sm.sg[tid];
    float tail = 0.f;
    if (tid == n - 1)
      for (int t = n; t < CH; ++t) tail += sm.sg[t];
    if (tid < n) a.dG[tok0 + t0 + tid] = v + tail;
  }
}

// ---------------------------------------------------------------------------
// Back through the write gains with a statistic and the decay.  Thread d owns
// key channel d.
template <typename E, int DK, int GAIN, bool CHAN>
__global__ __launch_bounds__(DK) void gain_bwd_kernel(GainBwdArgs a) {
  constexpr int NW = DK / 64;
  constexpr bool PG = GAIN == GAIN_PGDN, KD = GAIN == GAIN_KDN, ISO = GAIN == GAIN_KDN_ISO;
  constexpr bool ST = PG || KD;  // a per-channel statistic, recomputed per chunk
  __shared__ float red[4][NW];
  __shared__ float As[ST ? CH : 1][ST ? DK : 1];    // PGDN: A_t; KDN: p before token t
  __shared__ float iso[ISO ? 3 : 1][ISO ? CH : 1];  // KDN_ISO: b before token t, a_t, ||k_t||^2
  DN_LDS_POISON(red, sizeof(red));
  DN_LDS_POISON(As, sizeof(As));
  DN_LDS_POISON(iso, sizeof(iso));
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
      if constexpr (PG) {
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

// N consecutive fp32 or io elements from element offset `off` (16-byte
// accesses; off and N multiples of 8)
template <typename E, int N>
__device__ __forceinline__ void load_row(const void* base, long off, float (&v)[N]) {
  load_vec<E, N>(base, off, true, v);
}
template <int N>
__device__ __forceinline__ void store_row(float* base, long off, const float (&v)[N]) {
  f32x4* p = reinterpret_cast<f32x4*>(base + off);
#pragma unroll
  for (int i = 0; i < N / 4; ++i) p[i] = f32x4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
}

// Back through the gains without a statistic (KLA, GDN, explicit w),
// token-parallel: one workgroup per chunk of 64 tokens, four threads per
// token with a quarter of the key channels each; the sums over a token's
// channels are sums over its four lanes.  The decay's gradient is the suffix
// sum of dL/dG over the chunk's tokens: one wavefront's for scalar decay, per
// channel through LDS for per-channel decay.  Same derivatives as
// gain_bwd_kernel, summed in another order.
template <typename E, int DK, int GAIN, bool CHAN>
__global__ __launch_bounds__(4 * CH) void gain_bwd_tok_kernel(GainBwdArgs a) {
  constexpr int DQ = DK / 4;
  __shared__ float s_dg[CHAN ? CH * DK : 1];
  __shared__ float s_al[CHAN ? CH * DK : 1];
  DN_LDS_POISON(s_dg, sizeof(s_dg));
  DN_LDS_POISON(s_al, sizeof(s_al));
  const int T = a.T, nch = (T + CH - 1) / CH;
  const long bh = blockIdx.x / nch;
  const int c = static_cast<int>(blockIdx.x % nch);
  const int t0 = c * CH, n = min(CH, T - t0);
  const int tid = threadIdx.x, tl = tid >> 2, q = tid & 3, d0 = q * DQ;
  const bool ok = tl < n;
  const long ti = bh * T + t0 + tl;
  if (ok) {
    float dw[DQ];
    load_row<float, DQ>(a.dw_acc, ti * DK + d0, dw);
    if constexpr (GAIN == GAIN_EXPLICIT) {
      store_row<DQ>(a.dw_out, ti * DK + d0, dw);
    } else {
      float kv[DQ], dk[DQ];
      load_row<E, DQ>(a.k, ti * DK + d0, kv);
      load_row<float, DQ>(a.dk_out, ti * DK + d0, dk);
      // (the four lanes of a token share `ok`, so its lane sums stay inside it)
      float db = 0.f, n2 = 0.f;
#pragma unroll
      for (int i = 0; i < DQ; ++i) {
        db = fmaf(dw[i], kv[i], db);
        n2 = fmaf(kv[i], kv[i], n2);
      }
      db += __shfl_xor(db, 1);
      db += __shfl_xor(db, 2);
      const float et = a.g.eta[ti];
      if constexpr (GAIN == GAIN_KLA) {
        // w = beta k, beta = eta / (n + eps), n = ||k||^2
        n2 += __shfl_xor(n2, 1);
        n2 += __shfl_xor(n2, 2);
        const float den = n2 + a.g.eps, beta = et / den, g2 = db * (-et / (den * den));
#pragma unroll
        for (int i = 0; i < DQ; ++i) dk[i] = fmaf(beta, dw[i], fmaf(2.f * kv[i], g2, dk[i]));
        if (q == 0) a.deta[ti] = db / den;
      } else {
#pragma unroll
        for (int i = 0; i < DQ; ++i) dk[i] = fmaf(et, dw[i], dk[i]);
        if (q == 0) a.deta[ti] = db;
      }
      store_row<DQ>(a.dk_out, ti * DK + d0, dk);
    }
  }
  // dL/dalpha_t = (sum of dL/dG_j over j >= t in the chunk) / alpha_t
  if constexpr (CHAN) {
    if (ok) {
      float g[DQ], al[DQ];
      load_row<float, DQ>(a.dG, ti * DK + d0, g);
      load_row<E, DQ>(a.g.alpha, ti * DK + d0, al);
#pragma unroll
      for (int i = 0; i < DQ; ++i) {
        s_dg[tl * DK + d0 + i] = g[i];
        s_al[tl * DK + d0 + i] = al[i];
      }
    }
    __syncthreads();
    if (tid < DK) {
      float sfx = 0.f;
      for (int t = n - 1; t >= 0; --t) {
        sfx += s_dg[t * DK + tid];
        a.dalpha[(bh * T + t0 + t) * DK + tid] = sfx / s_al[t * DK + tid];
      }
    }
  } else if (tid < 64) {
    // lane l: token n - 1 - l, so that a prefix sum over the lanes is the
    // suffix sum over the tokens
    const int t = n - 1 - tid;
    float sfx = t >= 0 ? a.dG[bh * T + t0 + t] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(sfx, off);
      if (tid >= off) sfx += y;
    }
    if (t >= 0) a.dalpha[bh * T + t0 + t] = sfx / static_cast<const float*>(a.g.alpha)[bh * T + t0 + t];
  }
}

__global__ void zero_kernel(float* p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0.f;
}

}  // namespace bwd

template <typename E, int DK, bool CHAN, int DVS>
static hipError_t launch_bwd_state_w(const BwdArgs& a, hipStream_t st) {
  using Sm = bwd::Smem<E, DK, CHAN, DVS>;
  static_assert(sizeof(Sm) <= 160 * 1024, "LDS budget");
  if (a.dv % Sm::DVS != 0) return hipErrorInvalidValue;
  auto kern = bwd::chunk_bwd_state_kernel<E, DK, CHAN, DVS>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(sizeof(Sm)));
  if (err != hipSuccess) return err;
  const unsigned grid = static_cast<unsigned>(static_cast<long>(a.B) * a.H * (a.dv / Sm::DVS));
  hipLaunchKernelGGL(kern, dim3(grid), dim3(bwd::NT), sizeof(Sm), st, a);
  return hipGetLastError();
}

// Value slices of 32 columns, or of 16 (channel decay; and scalar decay when
// 32-column slices would leave most compute units idle: a workgroup's time
// is a serial walk over the chunks, so more, narrower slices finish sooner
// as long as they fit on the device at once)
constexpr long BWD_CU_COUNT = 256;  // compute units of an MI355X
template <typename E, int DK, bool CHAN>
static hipError_t launch_bwd_state_t(const BwdArgs& a, hipStream_t st) {
  if constexpr (CHAN) {
    return launch_bwd_state_w<E, DK, CHAN, 16>(a, st);
  } else {
    const long wide = static_cast<long>(a.B) * a.H * (a.dv / 32);
    if (2 * wide <= BWD_CU_COUNT) return launch_bwd_state_w<E, DK, CHAN, 16>(a, st);
    return launch_bwd_state_w<E, DK, CHAN, 32>(a, st);
  }
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

template <class Sm, class K>
static hipError_t launch_lds(K kern, unsigned grid, const BwdArgs& a, hipStream_t st, int threads = bwd::NT) {
  static_assert(sizeof(Sm) <= 160 * 1024, "LDS budget");
  const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             static_cast<int>(sizeof(Sm)));
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), sizeof(Sm), st, a);
  return hipGetLastError();
}
// Z and P for every chunk, the serial sweep in 64-column value slices, the
// tile kernel one workgroup per chunk
template <int DK>
static hipError_t launch_bwd_split_t(const BwdArgs& a, hipStream_t st, int part) {
  const long bh = static_cast<long>(a.B) * a.H;
  const long nch = (a.T + bwd::CH - 1) / bwd::CH;
  if (a.dv % bwd::DVS_S != 0 || a.Z_ck == nullptr || a.dS_ck == nullptr || a.nseg < 1 || a.nseg > nch ||
      (a.nseg > 1 && (a.segA == nullptr || a.segB == nullptr || a.seg_in == nullptr)))
    return hipErrorInvalidValue;
  if (part == 1) {
    hipError_t err =
        launch_lds<bwd::SmemZ<DK>>(bwd::chunk_bwd_zp_kernel<DK>, static_cast<unsigned>(bh * nch), a, st);
    if (err != hipSuccess) return err;
    const unsigned nv = static_cast<unsigned>(bh * a.nseg * (a.dv / bwd::DVS_S));
    if (a.nseg > 1) {
      // every segment's affine map, then the maps chained from dS_T (which
      // also gives dS0), then every segment from its own dS_out
      err = launch_lds<bwd::SmemS<DK>>(bwd::chunk_bwd_ds_kernel<DK, true>,
                                       nv + static_cast<unsigned>(bh * a.nseg * (DK / bwd::DVS_S)), a, st, bwd::NTS);
      if (err != hipSuccess) return err;
      CombineArgs ca;
      ca.B = a.B;
      ca.H = a.H;
      ca.nseg = a.nseg;
      ca.dk = DK;
      ca.dv = a.dv;
      ca.A = a.segA;
      ca.Bs = a.segB;
      ca.S0 = a.dS_T;
      ca.S_in = a.seg_in;
      ca.S_final = a.dS0;
      if ((err = launch_segment_combine(ca, st)) != hipSuccess) return err;
    }
    return launch_lds<bwd::SmemS<DK>>(bwd::chunk_bwd_ds_kernel<DK, false>, nv, a, st, bwd::NTS);
  }
  const unsigned gt = static_cast<unsigned>(bh * nch);
  if (a.fuse_gain == FUSE_KLA) return launch_lds<bwd::SmemT<DK>>(bwd::chunk_bwd_tiles_kernel<DK, FUSE_KLA>, gt, a, st);
  if (a.fuse_gain == FUSE_GDN) return launch_lds<bwd::SmemT<DK>>(bwd::chunk_bwd_tiles_kernel<DK, FUSE_GDN>, gt, a, st);
  return launch_lds<bwd::SmemT<DK>>(bwd::chunk_bwd_tiles_kernel<DK, FUSE_NONE>, gt, a, st);
}

hipError_t launch_chunk_bwd_split(const BwdArgs& a, hipStream_t st, int part) {
  if (a.T == 0 || a.B * a.H == 0) return hipSuccess;
  if (a.dk == 128) return launch_bwd_split_t<128>(a, st, part);
  if (a.dk == 64) return launch_bwd_split_t<64>(a, st, part);
  return hipErrorInvalidValue;
}

template <typename E, int DK, bool CHAN>
static hipError_t launch_gain_bwd_t(const GainBwdArgs& a, int gain, hipStream_t st) {
  if (gain == GAIN_KLA || gain == GAIN_GDN || gain == GAIN_EXPLICIT) {
    // token-parallel, one workgroup per chunk of 64 tokens
    const long nch = (a.T + bwd::CH - 1) / bwd::CH;
    if (nch == 0) return hipSuccess;
    const dim3 tg(static_cast<unsigned>(static_cast<long>(a.B) * a.H * nch)), tb(4 * bwd::CH);
    if (gain == GAIN_KLA)
      hipLaunchKernelGGL((bwd::gain_bwd_tok_kernel<E, DK, GAIN_KLA, CHAN>), tg, tb, 0, st, a);
    else if (gain == GAIN_GDN)
      hipLaunchKernelGGL((bwd::gain_bwd_tok_kernel<E, DK, GAIN_GDN, CHAN>), tg, tb, 0, st, a);
    else
      hipLaunchKernelGGL((bwd::gain_bwd_tok_kernel<E, DK, GAIN_EXPLICIT, CHAN>), tg, tb, 0, st, a);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>(a.B * a.H)), block(DK);
  switch (gain) {
#define DN_GAIN_BWD_CASE(G)                                                               \
  case G:                                                                                 \
    hipLaunchKernelGGL((bwd::gain_bwd_kernel<E, DK, G, CHAN>), grid, block, 0, st, a); \
    break;
    DN_GAIN_BWD_CASE(GAIN_PGDN)
    DN_GAIN_BWD_CASE(GAIN_KDN)
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
