// Chunked forward of the gated delta-rule recurrence on gfx950.
//
// One workgroup owns one (batch, head) and a slice of BV value columns; it
// walks the sequence in chunks of C = 64 tokens and keeps its d_k x BV slice
// of the fp32 state in registers for the whole sequence.  Value columns of S
// evolve independently (the residual e_t is per column, and every column
// shares the same key-space write: Kalman Delta Networks §2.1), so slices of
// one head need no communication.
//
// Chunk form (our statement of Kaczmarz Linear Attention §2.5 Eqs. 7-9 and
// Preconditioned DeltaNet §2.6 Eq. 6, extended to per-channel decay).  With
// G_t the cumulative log-decay inside the chunk and g_t = exp(G_t):
//
//   khat_i = g_i * k_i,  qhat_i = g_i * q_i,  wchk_j = w_j / g_j,
//   wtil_j = (g_n / g_j) * w_j
//   L = strict_lower(Khat Wchk^T),   M = lower_incl(Qhat Wchk^T)
//   (I + L) U = V - Khat S_in        (row i of U is the residual e_i)
//   O = Qhat S_in + M U,             S_out = diag(g_n) S_in + Wtil^T U
//
// Per chunk, in this order (barriers between the numbered steps):
//   1. the chunk's k, q, v slice and gates move from staging registers (loaded
//      from HBM during the previous chunk) into LDS, the next chunk's loads
//      are issued, and the previous chunk's output tile is stored;
//   2. gains: write vectors w_t (KLA/GDN/PGDN/KDN/explicit) and cumulative
//      log2-decay; the PGDN statistic A and the KDN variance p are carried
//      across chunks in registers of the thread owning the key channel;
//   3. the transposed write operand Wtil^T;
//   4. L and M as lower-triangular 16x16 tile pairs on the matrix cores;
//   5. each wavefront inverts one 16x16 diagonal block of I + L (fp32
//      forward substitution) and forms Khat S and Qhat S for its 16 value
//      columns;
//   6. per wavefront: blocked forward substitution
//      U_b = T_bb (R_b - sum_{m<b} L_bm U_m), O = Qhat S + M U and
//      S = diag(g_n) S + Wtil^T U.  With bf16 operands the solve and M U run
//      on 16x16x16 MFMAs whose B operand is the accumulator layout of U, so U
//      never leaves registers;
//   7. the output tile is staged in LDS and leaves in 16-byte rows at the
//      start of the next chunk.
// Operands are bf16 (fp32 for fp32 io) with fp32 accumulation; S, the
// diagonal-block inverses and all gain arithmetic stay fp32.
//
// Scalar decay: decay factors exp(G_i - G_j) are applied per element to the
// products of the raw k, q and w (no overflow for any decay).  Channel decay:
// khat, qhat and wchk are referenced to the chunk midpoint, which keeps each
// factor within exp of the decay accumulated over 32 tokens.
#include "common.hpp"
#include "gains.hpp"
#include "launch.hpp"

namespace dn {

constexpr int CH = 64;  // chunk length

// Synchronisation of LDS traffic between lanes of one wavefront: LDS
// instructions of a wavefront complete in order; the fences keep the
// compiler from moving LDS accesses across this point.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Hardware exp2 / log2 (v_exp_f32, v_log_f32).  Arguments here are decay
// sums and their differences (finite, and exp2 of very negative values
// underflowing to 0 is the right limit).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Channel decay: the scale 2^Gmid of the state rows, Gmid the log2-decay from
// the chunk start to its midpoint (token 31) and Gn to its end.  Referred to
// the midpoint, every operand factor stays within 2^96 and the scaled state
// stays normal while both half-chunk decays are at least 2^-96; beyond that
// the chunk form cannot be evaluated this way: a NaN scale turns the head's
// state and later outputs into NaN, and the head is flagged (*oor) for the
// tokenwise pass, which recomputes it.
__device__ __forceinline__ float midpoint_scale(float gm, float gn, int* oor) {
  const bool ok = gm >= -96.f && gn - gm >= -96.f;
  if (!ok) *oor = 1;
  return ok ? fast_exp2(gm) : __builtin_nanf("");
}
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// PGDN write scale B(A) = exp(-ln(x) s), s = r / (1 + |r|), r = ln A - mu
// (Preconditioned DeltaNet §2.4, Eq. 9) on the hardware log2 / rcp / exp2.
__device__ __forceinline__ float pgdn_scale_fast(float A, float mu, float log2x) {
  const float r = fast_log2(A) * 0.69314718055994531f - mu;
  const float sft = r * __builtin_amdgcn_rcpf(1.0f + fabsf(r));
  return fast_exp2(-log2x * sft);
}

// bf16 16x16x16 MFMA pieces.  Lane l: A row l % 16, k = 4 (l / 16) .. +3;
// B column l % 16, k = 4 (l / 16) .. +3; accumulator rows 4 (l / 16) .. +3 of
// column l % 16.  The accumulator of one product is therefore, packed to
// bf16, directly the B operand of the next.
__device__ __forceinline__ s16x4 frag16(const uint16_t* p, int ld, int lane) {
  return __builtin_bit_cast(
      s16x4, *reinterpret_cast<const u32x2*>(p + (lane & 15) * ld + 4 * (lane >> 4)));
}
__device__ __forceinline__ s16x4 pack16(f32x4 c) {
  const u32x2 v = {pack_bf2(c[0], c[1]), pack_bf2(c[2], c[3])};
  return __builtin_bit_cast(s16x4, v);
}
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Four consecutive rows r0 .. r0 + 3 of column cb + lane of a row-major bf16
// tile of pitch ld, as fp32, in one ds_read_b64_tr_b16: within each group of
// 16 lanes, lane l receives element l % 4 of the 8-byte piece addressed by
// lane 4 j + l / 4, so lane 4 j + q addresses row r0 + j, columns
// cb + 16 g + 4 q .. +3 (g = lane / 16) and every lane gets its own column.
typedef short s16x4_lds __attribute__((ext_vector_type(4), address_space(3)));
__device__ __forceinline__ f32x4 col4(const uint16_t* base, int ld, int r0, int cb, int lane) {
  const int a = lane & 15;
  const uint16_t* p = base + (r0 + (a >> 2)) * ld + cb + 16 * (lane >> 4) + 4 * (a & 3);
  const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_lds*)p));
  return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u),
               __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xFFFF0000u)};
}

template <typename E> struct Pad;
template <> struct Pad<uint16_t> { static constexpr int v = 8; };
template <> struct Pad<float> { static constexpr int v = 4; };

template <typename E, int DK, int BV, bool HAS_W>
struct ChunkSmem {
  static constexpr int PAD = Pad<E>::v;
  static constexpr int PK = DK + PAD;     // pitch of [token][d_k] operands
  static constexpr int PT = CH + PAD;     // pitch of [*][token] operands
  static constexpr int P16 = 16 + PAD;    // pitch of 16-wide blocks
  static constexpr int NW = BV / 16;
  alignas(16) E k[CH * PK];              // raw k (scalar decay) or khat (channel decay)
  alignas(16) E q[CH * PK];              // raw q or qhat
  alignas(16) E w[HAS_W ? CH * PK : 8];  // B operand of L, M: raw w (scalar) or wchk
  alignas(16) E wt[DK * PT];             // Wtil^T: [d][t]; stages channel alpha first
  alignas(16) E v[CH * BV];              // value slice [t][c]
  alignas(16) E lm[2 * CH * PT];         // -L (strictly lower) and M (lower incl.
                                         // diagonal), [i][j]; stages KDN omega first
  alignas(16) E tb[4 * 16 * P16];        // inverses of the diagonal blocks of I + L
  alignas(16) E sb[NW * 16 * PK];        // per wave: its 16 state columns, [c][d]
  alignas(16) E ub[NW * 16 * PT];        // per wave: U columns, [c][t]
  alignas(16) E xb[NW * 16 * P16];       // per wave: right-hand side of one block solve
  alignas(16) E o[CH * BV];              // output tile [t][c]
  alignas(16) float ld[4 * 16 * 16];     // diagonal 16x16 blocks of L, fp32
  alignas(16) float g2[CH];              // scalar decay: cumulative log2-decay
  alignas(16) float gam[CH];             // scalar decay: 2^g2
  alignas(16) float ah[DK];              // PGDN: statistic after the first half-chunk
  alignas(16) float aprod[CH];           // PGDN: prefix products of alphaP over the second half
  alignas(16) float acarry[DK];          // PGDN: statistic carried between chunks
  alignas(16) float gmid[DK];            // channel decay: 2^Gmid per channel
  alignas(16) float gn[DK];              // channel decay: 2^Gn per channel
  float cs[CH];                          // column scale of the L, M products
  float eta[CH], alpha[CH], ap[CH], bp[CH], mur[CH], r[CH];
  float zp[4][CH];                       // KDN: per-wavefront partial sums of z_t
  float pmid[DK], g31[DK];               // KDN, two segments: variance and log-decay after token 31
  float pcar[DK], g63[DK];               //   and after token 63 (the carry)
  float red[CH];                         // KDN: 1 / (r_t + z_t)
  int oor;                               // channel decay: a chunk beyond the chunk form's range
};

template <typename E, int DK, int BV, int GAIN, bool CHANNEL>
__global__ __launch_bounds__(BV * 4) __attribute__((amdgpu_waves_per_eu(1, 1)))
void chunk_fwd_kernel(ChunkArgs a) {
  constexpr int NW = BV / 16;
  constexpr int NT = 64 * NW;
  constexpr bool BF16 = sizeof(E) == 2;
  constexpr bool HAS_W = CHANNEL || GAIN == GAIN_PGDN || GAIN == GAIN_KDN || GAIN == GAIN_EXPLICIT;
  // PGDN with scalar decay: the statistic scan is split in two half-chunks
  // over 2 DK threads and the transcendental work is spread over all of them
  constexpr bool PG2 = GAIN == GAIN_PGDN && !CHANNEL && NT >= 2 * DK;
  constexpr bool SCAN = CHANNEL || (GAIN == GAIN_PGDN && !PG2) || GAIN == GAIN_KDN;
  // bf16 KDN with channel decay, one key channel per thread: the scans, the
  // z sums and the operand rescaling read four tokens of a channel per
  // transposing LDS read (col4) instead of one element at a time
  constexpr bool FASTCD = BF16 && CHANNEL && GAIN == GAIN_KDN && DK <= NT && DK % 64 == 0;
  // with 2 d_k threads, two per channel: segment 0 (tokens 0..31) scans the
  // variance from the carry while segment 1 (tokens 32..63) forms its decay
  // prefix, then segment 1 replays its variance scan from segment 0's end;
  // the z sums and the operands use all threads
  constexpr bool FASTCD2 = FASTCD && NT == 2 * DK;
  constexpr int HT = CH / 2;
  using Sm = ChunkSmem<E, DK, BV, HAS_W>;
  constexpr int PK = Sm::PK, PT = Sm::PT, P16 = Sm::P16;
  constexpr int VEC = 16 / sizeof(E);            // elements per 16-byte access
  constexpr int KV_LOADS = CH * DK / (NT * VEC); // 16-byte loads per thread (k or q)
  constexpr int V_LOADS = (CH * BV + NT * VEC - 1) / (NT * VEC);
  constexpr int CPT = (DK + NT - 1) / NT;        // key channels per thread
  constexpr int KS = DK / MmaK<E>::v;            // k-steps of a d_k contraction
  static_assert(KV_LOADS * NT * VEC == CH * DK, "k/q tile split");
  using EL = Elem<E>;
  using MM = Mma<E>;
  using Frag = typename MM::Frag;

  extern __shared__ __align__(16) unsigned char smem_raw[];
  DN_LDS_POISON(smem_raw, sizeof(Sm));
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);
  E* const sL = sm.lm;            // -L
  E* const sM = sm.lm + CH * PT;  // M

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g4 = lane >> 4, c16 = lane & 15;
  // XCD-aware mapping of the 1-D grid: consecutive workgroups are dealt to
  // the 8 XCDs in turn, so the value slices of one head get ids that are
  // equal modulo 8 and share that XCD's L2 (k and q are read once from HBM).
  const int ns = (a.dv + a.xcols) / BV;  // value slices (and transfer slices)
  const int nwg = ns * a.B * a.H;
  int bh, slice;
  {
    const int L = blockIdx.x;
    if (nwg % 8 == 0 && (nwg / 8) % ns == 0) {
      const int xcd = L % 8, r = L / 8;
      slice = r % ns;
      bh = xcd * (nwg / 8 / ns) + r / ns;
    } else {
      slice = L % ns;
      bh = L / ns;
    }
  }
  const int h = bh % a.H;
  const int col0 = slice * BV;  // first value column of this slice
  // a transfer slice: columns col0 - dv of S0 = I, v = 0, no output
  const bool xfer = col0 >= a.dv;
  const bool has_out = a.o && !xfer;
  const int T = a.T;
  const int nchunks = (T + CH - 1) / CH;
  const long qk_base = static_cast<long>(bh) * T * DK;
  const long v_base = static_cast<long>(bh) * T * a.dv;
  const E* gk = static_cast<const E*>(a.k) + qk_base;
  const E* gq = static_cast<const E*>(a.q) + qk_base;
  const E* gv = static_cast<const E*>(a.v) + v_base;
  E* go = a.o ? static_cast<E*>(a.o) + v_base : nullptr;

  // ---- state slice in registers: tile dt holds rows 16 dt + 4 g4 + i, column c16
  f32x4 S[DK / 16];
  {
    const int col = col0 + 16 * wave + c16;
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * dt + 4 * g4 + i;
        const float s0 = a.S0 && !xfer ? a.S0[(static_cast<long>(bh) * DK + row) * a.dv + col] : 0.f;
        S[dt][i] = xfer ? (row == col - a.dv ? 1.f : 0.f) : s0;
      }
  }
  // ---- per-channel gain state (PGDN statistic A, KDN variance p)
  float aux[CPT];
#pragma unroll
  for (int cc = 0; cc < CPT; ++cc) {
    const int d = tid + cc * NT;
    aux[cc] = (d < DK && a.aux0 && GAIN != GAIN_KDN_ISO) ? a.aux0[static_cast<long>(bh) * DK + d] : 1.f;
  }
  // isotropic KDN: the head's variance b, carried between chunks in LDS
  if constexpr (GAIN == GAIN_KDN_ISO) {
    if (tid == 0) sm.acarry[0] = a.aux0 ? a.aux0[bh] : 1.f;
  }
  if (tid == 0) sm.oor = 0;

  if constexpr (PG2) {
    if (tid < DK) sm.acarry[tid] = aux[0];
  }

  // ---- register staging of one chunk's inputs
  u32x4 pk[KV_LOADS], pq[KV_LOADS], pw[GAIN == GAIN_EXPLICIT ? KV_LOADS : 1];
  u32x4 pal[CHANNEL ? KV_LOADS : 1], pom[GAIN == GAIN_KDN ? KV_LOADS : 1];
  u32x4 pv[V_LOADS];
  float p_eta = 0.f, p_alpha = 1.f, p_ap = 1.f, p_bp = 0.f, p_r = 1.f;

  // Loads are unconditional: out-of-range tokens read row 0 of the chunk (in
  // range whenever the chunk exists) and are replaced by neutral values when
  // the registers are stashed into LDS, so no load result is consumed before
  // the next chunk.  A chunk is fetched in three parts issued at different
  // points of the previous chunk: part 0 = k (and explicit w, channel alpha),
  // 1 = q (and KDN omega), 2 = v and the per-token gates.
  auto fetch = [&](int c, int part) __attribute__((always_inline)) {
    const int t0 = c * CH;
    const int n = min(CH, T - t0);
    if (part < 2) {
#pragma unroll
      for (int j = 0; j < KV_LOADS; ++j) {
        const int e = (tid + j * NT) * VEC;  // element index inside the [CH][DK] tile
        const int t = e / DK, d = e % DK;
        const long off = static_cast<long>(t0 + (t < n ? t : 0)) * DK + d;
        if (part == 0) {
          pk[j] = *reinterpret_cast<const u32x4*>(gk + off);
          if constexpr (GAIN == GAIN_EXPLICIT)
            pw[j] = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.g.w) + qk_base + off);
          if constexpr (CHANNEL)
            pal[j] = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.g.alpha) + qk_base + off);
        } else {
          pq[j] = *reinterpret_cast<const u32x4*>(gq + off);
          if constexpr (GAIN == GAIN_KDN)
            pom[j] = *reinterpret_cast<const u32x4*>(static_cast<const E*>(a.g.omega) + qk_base + off);
        }
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < V_LOADS; ++j) {
      const int e = (tid + j * NT) * VEC;
      const int t = e / BV, cc = e % BV;
      const bool ok = e < CH * BV && t < n;
      // transfer slices read v = 0 (their columns lie past d_v: the load
      // takes column 0 and is discarded)
      const u32x4 ld = *reinterpret_cast<const u32x4*>(gv + static_cast<long>(t0 + (ok ? t : 0)) * a.dv +
                                                       (xfer ? 0 : col0) + (ok ? cc : 0));
      pv[j] = xfer ? u32x4{0u, 0u, 0u, 0u} : ld;
    }
    if (tid < CH) {
      const long ti = static_cast<long>(bh) * T + t0 + (tid < n ? tid : 0);
      if (GAIN != GAIN_KDN && GAIN != GAIN_EXPLICIT && GAIN != GAIN_KDN_ISO) p_eta = a.g.eta[ti];
      // isotropic KDN: the per-token process noise omega travels in the eta slot
      if (GAIN == GAIN_KDN_ISO) p_eta = static_cast<const float*>(a.g.omega)[ti];
      if (!CHANNEL) p_alpha = static_cast<const float*>(a.g.alpha)[ti];
      if (GAIN == GAIN_PGDN) {
        p_ap = a.g.alphaP[ti];
        p_bp = a.g.betaP[ti];
      }
      if (GAIN == GAIN_KDN || GAIN == GAIN_KDN_ISO) p_r = a.g.r[ti];
    }
  };

  // registers -> LDS for chunk c, substituting neutral values past the end:
  // k = q = v = w = omega = 0, alpha = alphaP = 1, betaP = eta = 0, r = 1
  auto stash = [&](int n) __attribute__((always_inline)) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < KV_LOADS; ++j) {
      const int e = (tid + j * NT) * VEC;
      const int t = e / DK, d = e % DK;
      const bool ok = t < n;
      *reinterpret_cast<u32x4*>(&sm.k[t * PK + d]) = ok ? pk[j] : z;
      *reinterpret_cast<u32x4*>(&sm.q[t * PK + d]) = ok ? pq[j] : z;
      if constexpr (GAIN == GAIN_EXPLICIT)
        *reinterpret_cast<u32x4*>(&sm.w[t * PK + d]) = ok ? pw[j] : z;
      if constexpr (CHANNEL) {
        const u32x4 one4 = BF16 ? u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}
                                : u32x4{0x3F800000u, 0x3F800000u, 0x3F800000u, 0x3F800000u};
        pal[j] = ok ? pal[j] : one4;
      }
      if constexpr (GAIN == GAIN_KDN) pom[j] = ok ? pom[j] : z;
    }
#pragma unroll
    for (int j = 0; j < V_LOADS; ++j) {
      const int e = (tid + j * NT) * VEC;
      if (e < CH * BV) *reinterpret_cast<u32x4*>(&sm.v[e]) = (e / BV < n) ? pv[j] : z;
    }
    if (tid < CH) {
      const bool ok = tid < n;
      const float r = ok ? p_r : 1.f;
      sm.eta[tid] = ok ? p_eta : 0.f;
      sm.alpha[tid] = ok ? p_alpha : 1.f;
      sm.ap[tid] = ok ? p_ap : 1.f;
      sm.bp[tid] = ok ? p_bp : 0.f;
      sm.r[tid] = r;
      sm.mur[tid] = a.g.mu_info / r;
    }
  };

  // output tile of a chunk (in sm.o) -> HBM, 16-byte rows
  auto store_out = [&](int ts, int nn) __attribute__((always_inline)) {
    if (!has_out) return;  // a transfer slice, or o == NULL
    for (int e = tid * VEC; e < CH * BV; e += NT * VEC) {
      const int t = e / BV, cc = e % BV;
      if (t < nn)
        *reinterpret_cast<u32x4*>(go + static_cast<long>(ts + t) * a.dv + col0 + cc) =
            *reinterpret_cast<const u32x4*>(&sm.o[e]);
    }
  };

  if (nchunks > 0) {
    fetch(0, 0);
    fetch(0, 1);
    fetch(0, 2);
  }

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * CH;
    const int n = min(CH, T - t0);
    stash(n);
    // per-channel gates of this chunk, consumed in step 2
    u32x4 cal[CHANNEL ? KV_LOADS : 1], com[GAIN == GAIN_KDN ? KV_LOADS : 1];
#pragma unroll
    for (int j = 0; j < (CHANNEL ? KV_LOADS : 0); ++j) cal[j] = pal[j];
#pragma unroll
    for (int j = 0; j < (GAIN == GAIN_KDN ? KV_LOADS : 0); ++j) com[j] = pom[j];
    __syncthreads();  // (A) chunk inputs visible
    // the next chunk's inputs travel from HBM while this chunk is processed;
    // the previous chunk's output tile leaves after them, so that waiting for
    // these loads at the next stash never waits on the stores
    if (c + 1 < nchunks) fetch(c + 1, 0);
    if (c > 0) store_out(t0 - CH, CH);

    // ================= 2. gains =================
    if constexpr (!CHANNEL) {
      // cumulative log2-decay by a wavefront inclusive scan; tokens >= n have alpha = 1
      if (wave == NW - 1) {
        float x = fast_log2(sm.alpha[lane]);
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(x, off, 64);
          if (lane >= off) x += y;
        }
        sm.g2[lane] = x;
        sm.gam[lane] = fast_exp2(x);
        if constexpr (PG2) {
          // prefix products of alphaP over tokens 32..63
          float pr = lane >= CH / 2 ? sm.ap[lane] : 1.f;
#pragma unroll
          for (int off = 1; off < CH / 2; off <<= 1) {
            const float y = __shfl_up(pr, off, 64);
            if (lane - off >= CH / 2) pr *= y;
          }
          sm.aprod[lane] = pr;
        }
      }
    }
    if constexpr (PG2) {
      // half 0 (tokens 0..31) starts from the carried statistic, half 1
      // (tokens 32..63) from 0; half 1 adds aprod_t * A_31 afterwards
      constexpr int HT = CH / 2;
      const int d = tid % DK, half = tid / DK;
      float A[HT];
      if (tid < 2 * DK) {
        float st = half == 0 ? sm.acarry[d] : 0.f;
#pragma unroll
        for (int i = 0; i < HT; ++i) {
          const int t = half * HT + i;
          st = pgdn_stat(st, sm.ap[t], sm.bp[t], EL::get(sm.k[t * PK + d]));
          A[i] = st;
        }
        if (half == 0) sm.ah[d] = st;
      }
      __syncthreads();
      if (tid < 2 * DK) {
        const float base = half == 1 ? sm.ah[d] : 0.f;
        const float mu = a.g.mu_log[h];
        float At = 0.f;
#pragma unroll
        for (int i = 0; i < HT; ++i) {
          const int t = half * HT + i;
          At = half == 1 ? fmaf(sm.aprod[t], base, A[i]) : A[i];
          const float kk = EL::get(sm.k[t * PK + d]);
          sm.w[t * PK + d] = EL::put(sm.eta[t] * pgdn_scale_fast(At, mu, a.g.log2x) * kk);
        }
        if (half == 1) sm.acarry[d] = At;
      }
    }
    if constexpr (GAIN == GAIN_KLA || GAIN == GAIN_GDN || GAIN == GAIN_KDN_ISO) {
      // ||k_t||^2 (KLA, isotropic KDN) with NT/64 threads per token, 16-byte
      // LDS reads; column scale beta_t (isotropic KDN: ||k_t||^2 kept for its
      // variance scan below)
      constexpr int TPT = NT / CH;
      const int t = tid / TPT, part = tid % TPT;
      float s = 0.f;
      if (GAIN == GAIN_KLA || GAIN == GAIN_KDN_ISO) {
        constexpr int PER = DK / TPT;
#pragma unroll
        for (int d0 = 0; d0 < PER; d0 += VEC) {
          const u32x4 raw = *reinterpret_cast<const u32x4*>(&sm.k[t * PK + part * PER + d0]);
          if constexpr (BF16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float lo = __uint_as_float(raw[i] << 16);
              const float hi = __uint_as_float(raw[i] & 0xFFFF0000u);
              s = fmaf(lo, lo, s);
              s = fmaf(hi, hi, s);
            }
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float x = __uint_as_float(raw[i]);
              s = fmaf(x, x, s);
            }
          }
        }
#pragma unroll
        for (int off = 1; off < TPT; off <<= 1) s += __shfl_xor(s, off, 64);
      }
      if (part == 0) {
        if constexpr (GAIN == GAIN_KDN_ISO) sm.zp[0][t] = s;
        else sm.cs[t] = (GAIN == GAIN_KLA) ? kla_beta(sm.eta[t], s, a.g.eps) : sm.eta[t];
      }
    }
    if constexpr (GAIN == GAIN_PGDN || GAIN == GAIN_KDN || GAIN == GAIN_EXPLICIT) {
      if (tid < CH) sm.cs[tid] = 1.f;
    }

    // per-channel scans: channel decay G, PGDN statistic A, KDN variance p.
    // Threads own key channels; the carried A / p live in their registers.
    float gch[CHANNEL ? CPT : 1][CHANNEL ? CH : 1];
    float pkr[GAIN == GAIN_KDN ? CPT : 1][GAIN == GAIN_KDN ? CH : 1];  // KDN: p_hat * k
    float gs[FASTCD2 ? HT : 1], ps[FASTCD2 ? HT : 1];  // two segments: G and p_hat * k of 32 tokens
    const int seg = tid / DK, dch = tid % DK, cbs = 64 * (dch / 64), tbs = seg * HT;
    if constexpr (SCAN) {
      E* s_al = sm.wt;  // channel alpha staged as [t][d] (wt is built after barrier B)
      E* s_om = sm.lm;  // KDN omega staged as [t][d] (lm is built after barrier C)
      if constexpr (CHANNEL || GAIN == GAIN_KDN) {
#pragma unroll
        for (int j = 0; j < KV_LOADS; ++j) {
          const int e = (tid + j * NT) * VEC;
          if constexpr (CHANNEL) *reinterpret_cast<u32x4*>(&s_al[e]) = cal[j];
          if constexpr (GAIN == GAIN_KDN) *reinterpret_cast<u32x4*>(&s_om[e]) = com[j];
        }
        __syncthreads();
      }
      const float mu = GAIN == GAIN_PGDN ? a.g.mu_log[h] : 0.f;
      if constexpr (FASTCD2) {
        const uint16_t* al16 = reinterpret_cast<const uint16_t*>(s_al);
        const uint16_t* om16 = reinterpret_cast<const uint16_t*>(s_om);
        const uint16_t* k16 = reinterpret_cast<const uint16_t*>(sm.k);
        float G = 0.f, st = aux[0];
#pragma unroll
        for (int t4 = 0; t4 < HT; t4 += 4) {
          const f32x4 al = col4(al16, DK, tbs + t4, cbs, lane);
          if (seg == 0) {
            const f32x4 om = col4(om16, DK, t4, cbs, lane);
            const f32x4 kk = col4(k16, PK, t4, cbs, lane);
            const f32x4 mr = *reinterpret_cast<const f32x4*>(&sm.mur[t4]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float ph = kdn_predict(al[j], st, om[j]);
              ps[t4 + j] = ph * kk[j];
              st = kdn_update(ph, kk[j], mr[j]);
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            G += fast_log2(al[j]);
            gs[t4 + j] = G;
          }
        }
        if (seg == 0) {
          sm.pmid[dch] = st;
          sm.g31[dch] = G;
        }
        __syncthreads();
        if (seg == 1) {
          const float g0 = sm.g31[dch];
          st = sm.pmid[dch];
#pragma unroll
          for (int t4 = 0; t4 < HT; t4 += 4) {
            const f32x4 al = col4(al16, DK, HT + t4, cbs, lane);
            const f32x4 om = col4(om16, DK, HT + t4, cbs, lane);
            const f32x4 kk = col4(k16, PK, HT + t4, cbs, lane);
            const f32x4 mr = *reinterpret_cast<const f32x4*>(&sm.mur[HT + t4]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float ph = kdn_predict(al[j], st, om[j]);
              ps[t4 + j] = ph * kk[j];
              st = kdn_update(ph, kk[j], mr[j]);
              gs[t4 + j] += g0;
            }
          }
          sm.pcar[dch] = st;
          sm.g63[dch] = gs[HT - 1];
        }
      } else if constexpr (FASTCD) {
        if (tid < DK) {  // wavefronts 0 .. DK / 64 - 1, channel = tid
          const int cb = 64 * wave;
          float G = 0.f, st = aux[0];
#pragma unroll
          for (int t4 = 0; t4 < CH; t4 += 4) {
            const f32x4 al = col4(reinterpret_cast<const uint16_t*>(s_al), DK, t4, cb, lane);
            const f32x4 om = col4(reinterpret_cast<const uint16_t*>(s_om), DK, t4, cb, lane);
            const f32x4 kk = col4(reinterpret_cast<const uint16_t*>(sm.k), PK, t4, cb, lane);
            const f32x4 mr = *reinterpret_cast<const f32x4*>(&sm.mur[t4]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              G += fast_log2(al[j]);
              gch[0][t4 + j] = G;
              const float ph = kdn_predict(al[j], st, om[j]);
              pkr[0][t4 + j] = ph * kk[j];
              st = kdn_update(ph, kk[j], mr[j]);
            }
          }
          aux[0] = st;
        }
      } else
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) {
        const int d = tid + cc * NT;
        if (d < DK) {
          float G = 0.f, st = aux[cc];
#pragma unroll
          for (int t = 0; t < CH; ++t) {
            const float al = CHANNEL ? EL::get(s_al[t * DK + d]) : sm.alpha[t];
            if constexpr (CHANNEL) {
              G += fast_log2(al);
              gch[cc][t] = G;
            }
            const float kk = EL::get(sm.k[t * PK + d]);
            if constexpr (GAIN == GAIN_PGDN) {
              st = pgdn_stat(st, sm.ap[t], sm.bp[t], kk);
              const float wv = sm.eta[t] * pgdn_scale(st, mu, a.g.log2x) * kk;
              sm.w[t * PK + d] = EL::put(wv);
            }
            if constexpr (GAIN == GAIN_KDN) {
              const float ph = kdn_predict(al, st, EL::get(s_om[t * DK + d]));
              pkr[cc][t] = ph * kk;
              st = kdn_update(ph, kk, sm.mur[t]);
            }
          }
          aux[cc] = st;
        }
      }
      if constexpr (GAIN == GAIN_KDN) {
        // z_t = sum_d p_hat k^2: per-wavefront sums (reduce-scattered, lane t
        // gets token t), combined over the wavefronts in a fixed order
        static_assert(CH == 64, "one token per lane");
        if constexpr (FASTCD2) {
          // z partial sums of this wavefront's 64 channels over its segment's
          // 32 tokens; lanes l < 32 get token tbs + l
          float zt[HT];
#pragma unroll
          for (int t4 = 0; t4 < HT; t4 += 4) {
            const f32x4 kk = col4(reinterpret_cast<const uint16_t*>(sm.k), PK, tbs + t4, cbs, lane);
#pragma unroll
            for (int j = 0; j < 4; ++j) zt[t4 + j] = ps[t4 + j] * kk[j];
          }
          const float zs = wave_reduce_scatter32(zt, lane);
          if (lane < HT) sm.zp[wave][lane] = zs;
          __syncthreads();
          if (tid < CH) {
            const int sg = tid / HT;
            float z = 0.f;
#pragma unroll
            for (int ww = 0; ww < DK / 64; ++ww) z += sm.zp[sg * (DK / 64) + ww][tid % HT];
            sm.red[tid] = 1.f / (sm.r[tid] + z);
          }
          if (seg == 0) aux[0] = sm.pcar[dch];  // the variance carried to the next chunk
        } else {
        float zt[CH];
        if constexpr (FASTCD) {
          if (tid < DK) {
#pragma unroll
            for (int t4 = 0; t4 < CH; t4 += 4) {
              const f32x4 kk = col4(reinterpret_cast<const uint16_t*>(sm.k), PK, t4, 64 * wave, lane);
#pragma unroll
              for (int j = 0; j < 4; ++j) zt[t4 + j] = pkr[0][t4 + j] * kk[j];
            }
          } else {
#pragma unroll
            for (int t = 0; t < CH; ++t) zt[t] = 0.f;
          }
        } else
#pragma unroll
        for (int t = 0; t < CH; ++t) {
          float z = 0.f;
#pragma unroll
          for (int cc = 0; cc < CPT; ++cc) {
            const int d = tid + cc * NT;
            if (d < DK) z += pkr[cc][t] * EL::get(sm.k[t * PK + d]);
          }
          zt[t] = z;
        }
        sm.zp[wave][lane] = wave_reduce_scatter64(zt, lane);
        __syncthreads();
        if (tid < CH) {
          float z = 0.f;
#pragma unroll
          for (int ww = 0; ww < NW; ++ww) z += sm.zp[ww][tid];
          sm.red[tid] = 1.f / (sm.r[tid] + z);
        }
        }
      }
    }
    if constexpr (GAIN == GAIN_KDN_ISO) {
      // isotropic KDN (Kalman Delta Networks §2.7, Eq. 40): the mean of
      // alpha_t^2 over the channels (channel decay: from its staged copy,
      // NT/64 threads per token), then one thread runs the head's variance
      // through the chunk and sets the column scales beta_t
      constexpr int TPT = NT / CH;
      const int t = tid / TPT, part = tid % TPT;
      float s2 = 0.f;
      if constexpr (CHANNEL) {
        constexpr int PER = DK / TPT;
        const E* s_al = sm.wt;
#pragma unroll
        for (int d0 = 0; d0 < PER; ++d0) {
          const float x = EL::get(s_al[t * DK + part * PER + d0]);
          s2 = fmaf(x, x, s2);
        }
#pragma unroll
        for (int off = 1; off < TPT; off <<= 1) s2 += __shfl_xor(s2, off, 64);
        s2 *= 1.0f / DK;
      } else {
        s2 = sm.alpha[t] * sm.alpha[t];
      }
      if (part == 0) sm.zp[1][t] = s2;
      __syncthreads();
      if (tid == 0) {
        float b = sm.acarry[0];
        for (int tt = 0; tt < CH; ++tt) {
          const float nk = sm.zp[0][tt], rr = sm.r[tt];
          const float bh_ = kdn_iso_predict(sm.zp[1][tt], b, sm.eta[tt]);
          sm.cs[tt] = kdn_iso_beta(bh_, rr, nk);
          b = kdn_iso_update(bh_, nk, a.g.mu_info / (DK * rr));
        }
        sm.acarry[0] = b;
      }
    }
    __syncthreads();  // (B) gains visible
    if (c + 1 < nchunks) fetch(c + 1, 1);

    // ================= 3. write-vector operands =================
    if constexpr (!CHANNEL) {
      if constexpr (GAIN == GAIN_KDN) {
#pragma unroll
        for (int cc = 0; cc < CPT; ++cc) {
          const int d = tid + cc * NT;
          if (d < DK)
#pragma unroll
            for (int t = 0; t < CH; ++t) sm.w[t * PK + d] = EL::put(pkr[cc][t] * sm.red[t]);
        }
        __syncthreads();
      }
      // Wtil^T[d][t] = 2^(G_{n-1} - G_t) w_t[d], in 4-token x VEC-channel blocks:
      // 16-byte row reads of w (or k), transposed 8/16-byte writes.
      const float gl = sm.g2[CH - 1];
      const E* src = HAS_W ? sm.w : sm.k;
      for (int blk = tid; blk < (CH / 4) * (DK / VEC); blk += NT) {
        const int tb4 = blk % (CH / 4), db = blk / (CH / 4);
        const int tt0 = 4 * tb4, dd0 = db * VEC;
        float val[4][VEC];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = tt0 + i;
          const float f = sm.cs[t] * fast_exp2(gl - sm.g2[t]);
          const u32x4 raw = *reinterpret_cast<const u32x4*>(&src[t * PK + dd0]);
          if constexpr (BF16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              val[i][2 * j] = f * __uint_as_float(raw[j] << 16);
              val[i][2 * j + 1] = f * __uint_as_float(raw[j] & 0xFFFF0000u);
            }
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) val[i][j] = f * __uint_as_float(raw[j]);
          }
        }
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          E* dst = &sm.wt[(dd0 + j) * PT + tt0];
          if constexpr (BF16) {
            const u32x2 p2 = {pack_bf2(val[0][j], val[1][j]), pack_bf2(val[2][j], val[3][j])};
            *reinterpret_cast<u32x2*>(dst) = p2;
          } else {
            const f32x4 v4 = {val[0][j], val[1][j], val[2][j], val[3][j]};
            *reinterpret_cast<f32x4*>(dst) = v4;
          }
        }
      }
    } else {
      // channel decay: rescale k, q in place to the chunk midpoint, build wchk and Wtil^T
      if constexpr (FASTCD2) {
        // thread (channel dch, segment seg): its 32 tokens; G at tokens 31
        // and 63 from the scan's boundary values
        const float gm = seg == 0 ? gs[HT - 1] : sm.g31[dch], gl = sm.g63[dch];
        if (seg == 0) {
          sm.gmid[dch] = midpoint_scale(gm, gl, &sm.oor);
          sm.gn[dch] = fast_exp2(gl);
        }
        const float fl = fast_exp2(gl - gm);  // 2^(Gn - Gmid)
#pragma unroll
        for (int t4 = 0; t4 < HT; t4 += 4) {
          const int tt = tbs + t4;
          const f32x4 kk = col4(reinterpret_cast<const uint16_t*>(sm.k), PK, tt, cbs, lane);
          const f32x4 qq = col4(reinterpret_cast<const uint16_t*>(sm.q), PK, tt, cbs, lane);
          const f32x4 rd = *reinterpret_cast<const f32x4*>(&sm.red[tt]);
          float wtv[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int t = tt + j;
            const float up = fast_exp2(gs[t4 + j] - gm), down = fast_exp2(gm - gs[t4 + j]);
            const float wv = ps[t4 + j] * rd[j];
            sm.k[t * PK + dch] = EL::put(up * kk[j]);
            sm.q[t * PK + dch] = EL::put(up * qq[j]);
            sm.w[t * PK + dch] = EL::put(down * wv);
            wtv[j] = fl * down * wv;  // 2^(Gn - G_t) w_t
          }
          *reinterpret_cast<u32x2*>(&sm.wt[dch * PT + tt]) = u32x2{pack_bf2(wtv[0], wtv[1]), pack_bf2(wtv[2], wtv[3])};
        }
      } else if constexpr (FASTCD) {
        if (tid < DK) {
          const int d = tid, cb = 64 * wave;
          const float gm = gch[0][CH / 2 - 1], gl = gch[0][CH - 1];
          sm.gmid[d] = midpoint_scale(gm, gl, &sm.oor);
          sm.gn[d] = fast_exp2(gl);
          const float fl = fast_exp2(gl - gm);  // 2^(Gn - Gmid)
#pragma unroll
          for (int t4 = 0; t4 < CH; t4 += 4) {
            const f32x4 kk = col4(reinterpret_cast<const uint16_t*>(sm.k), PK, t4, cb, lane);
            const f32x4 qq = col4(reinterpret_cast<const uint16_t*>(sm.q), PK, t4, cb, lane);
            const f32x4 rd = *reinterpret_cast<const f32x4*>(&sm.red[t4]);
            float wtv[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int t = t4 + j;
              const float up = fast_exp2(gch[0][t] - gm), down = fast_exp2(gm - gch[0][t]);
              const float wv = pkr[0][t] * rd[j];
              sm.k[t * PK + d] = EL::put(up * kk[j]);
              sm.q[t * PK + d] = EL::put(up * qq[j]);
              sm.w[t * PK + d] = EL::put(down * wv);
              wtv[j] = fl * down * wv;  // 2^(Gn - G_t) w_t
            }
            *reinterpret_cast<u32x2*>(&sm.wt[d * PT + t4]) = u32x2{pack_bf2(wtv[0], wtv[1]), pack_bf2(wtv[2], wtv[3])};
          }
        }
      } else
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) {
        const int d = tid + cc * NT;
        if (d < DK) {
          const float gm = gch[cc][CH / 2 - 1], gl = gch[cc][CH - 1];
          sm.gmid[d] = midpoint_scale(gm, gl, &sm.oor);
          sm.gn[d] = fast_exp2(gl);
#pragma unroll
          for (int t = 0; t < CH; ++t) {
            const float kk = EL::get(sm.k[t * PK + d]);
            float wv;
            if constexpr (GAIN == GAIN_KDN) wv = pkr[cc][t] * sm.red[t];
            else if constexpr (GAIN == GAIN_PGDN || GAIN == GAIN_EXPLICIT) wv = EL::get(sm.w[t * PK + d]);
            else wv = sm.cs[t] * kk;
            const float up = fast_exp2(gch[cc][t] - gm);
            sm.k[t * PK + d] = EL::put(up * kk);
            sm.q[t * PK + d] = EL::put(up * EL::get(sm.q[t * PK + d]));
            sm.w[t * PK + d] = EL::put(fast_exp2(gm - gch[cc][t]) * wv);
            sm.wt[d * PT + t] = EL::put(fast_exp2(gl - gch[cc][t]) * wv);
          }
        }
      }
    }
    __syncthreads();  // (C) operands of the intra-chunk products ready
    if (c + 1 < nchunks) fetch(c + 1, 2);

    // ================= 4. L and M, lower-triangular 16x16 tile pairs =================
    {
      const E* Bop = HAS_W ? sm.w : sm.k;
      for (int pair = wave; pair < 10; pair += NW) {
        int tt = pair, bi = 0;  // 0..9 -> (bi, bj), bj <= bi
        while (tt > bi) {
          tt -= bi + 1;
          ++bi;
        }
        const int bj = tt;
        // transposed tiles: C[j][i] = wchk_j . khat_i (qhat_i); lane (g4, c16)
        // then holds row i = 16 bi + c16, columns j = 16 bj + 4 g4 .. +3
        Frag fb[KS], fk[KS], fq[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          fb[s] = MM::frag(Bop + 16 * bj * PK, PK, lane, s);
          fk[s] = MM::frag(sm.k + 16 * bi * PK, PK, lane, s);
          fq[s] = MM::frag(sm.q + 16 * bi * PK, PK, lane, s);
        }
        f32x4 accL = zero4(), accM = zero4();
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          accL = MM::mma(fb[s], fk[s], accL);
          accM = MM::mma(fb[s], fq[s], accM);
        }
        const int i = 16 * bi + c16, j0 = 16 * bj + 4 * g4;
        f32x4 f = {1.f, 1.f, 1.f, 1.f};
        if constexpr (!CHANNEL) {
          const float gi = sm.g2[i];
          const f32x4 gj = *reinterpret_cast<const f32x4*>(&sm.g2[j0]);
          const f32x4 csj = *reinterpret_cast<const f32x4*>(&sm.cs[j0]);
#pragma unroll
          for (int u = 0; u < 4; ++u) f[u] = fast_exp2(gi - gj[u]) * csj[u];
        }
        f32x4 lv, mv;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          lv[u] = j0 + u < i ? accL[u] * f[u] : 0.f;
          mv[u] = j0 + u <= i ? accM[u] * f[u] : 0.f;
        }
        const f32x4 nl = (bi == bj) ? zero4() : -lv;
        if constexpr (BF16) {
          *reinterpret_cast<u32x2*>(&sM[i * PT + j0]) = u32x2{pack_bf2(mv[0], mv[1]), pack_bf2(mv[2], mv[3])};
          *reinterpret_cast<u32x2*>(&sL[i * PT + j0]) = u32x2{pack_bf2(nl[0], nl[1]), pack_bf2(nl[2], nl[3])};
        } else {
          *reinterpret_cast<f32x4*>(&sM[i * PT + j0]) = mv;
          *reinterpret_cast<f32x4*>(&sL[i * PT + j0]) = nl;
        }
        if (bi == bj) *reinterpret_cast<f32x4*>(&sm.ld[(bi * 16 + c16) * 16 + 4 * g4]) = lv;
      }
      // zero the strictly-upper tiles of -L and M
      for (int e = tid; e < 6 * 256; e += NT) {
        const int tile = e >> 8, w = e & 255;
        const int bi = tile < 3 ? 0 : (tile < 5 ? 1 : 2);
        const int bj = tile < 3 ? tile + 1 : (tile < 5 ? tile - 1 : 3);
        const int i = 16 * bi + (w >> 4), jj = 16 * bj + (w & 15);
        sL[i * PT + jj] = EL::put(0.f);
        sM[i * PT + jj] = EL::put(0.f);
      }
    }
    __syncthreads();  // (D) L, M ready

    // ================= 5. diagonal-block inverses and Khat S, Qhat S =================
    // wavefront w inverts diagonal block(s) w, w + NW, ...: lane c < 16
    // computes column c of (I + L_bb)^-1 by forward substitution (rows of
    // L_bb are broadcast LDS reads).
    for (int b = wave; b < 4; b += NW) {
      if (lane < 16) {
        const float* Lb = sm.ld + b * 256;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float row[16];
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 r4 = *reinterpret_cast<const f32x4*>(&Lb[i * 16 + 4 * q4]);
#pragma unroll
            for (int u = 0; u < 4; ++u) row[4 * q4 + u] = r4[u];
          }
          float s0 = (i == lane) ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
          for (int j = 0; j < i; ++j) {
            if (j & 1) s1 = fmaf(-row[j], x[j], s1);
            else s0 = fmaf(-row[j], x[j], s0);
          }
          x[i] = s0 + s1;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.tb[(b * 16 + i) * P16 + lane] = EL::put(x[i]);
      }
    }

    E* sb = sm.sb + wave * 16 * PK;
    E* ub = sm.ub + wave * 16 * PT;
    E* xb = sm.xb + wave * 16 * P16;
    // S columns -> [c][d] operand (channel decay: rows scaled by 2^Gmid)
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt) {
      f32x4 s4 = S[dt];
      if constexpr (CHANNEL) {
        const f32x4 gm = *reinterpret_cast<const f32x4*>(&sm.gmid[16 * dt + 4 * g4]);
        s4 = s4 * gm;
      }
      E* dst = &sb[c16 * PK + 16 * dt + 4 * g4];
      if constexpr (BF16) {
        const u32x2 p2 = {pack_bf2(s4[0], s4[1]), pack_bf2(s4[2], s4[3])};
        *reinterpret_cast<u32x2*>(dst) = p2;
      } else {
        *reinterpret_cast<f32x4*>(dst) = s4;
      }
    }
    wave_lds_sync();

    f32x4 R[4], O[4];
    {
      Frag fs[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) fs[s] = MM::frag(sb, PK, lane, s);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        Frag fk[KS], fq[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          fk[s] = MM::frag(sm.k + 16 * rt * PK, PK, lane, s);
          fq[s] = MM::frag(sm.q + 16 * rt * PK, PK, lane, s);
        }
        f32x4 kacc = zero4(), qacc = zero4();
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          kacc = MM::mma(fk[s], fs[s], kacc);
          qacc = MM::mma(fq[s], fs[s], qacc);
        }
        const f32x4 gt = *reinterpret_cast<const f32x4*>(&sm.gam[16 * rt + 4 * g4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 16 * rt + 4 * g4 + i;
          const float sc = CHANNEL ? 1.f : gt[i];
          R[rt][i] = EL::get(sm.v[t * BV + 16 * wave + c16]) - sc * kacc[i];
          O[rt][i] = sc * qacc[i];
        }
      }
    }
    __syncthreads();  // (E) block inverses ready

    // ================= 6. solve, output, state update (per wavefront) =================
    if constexpr (BF16) {
      s16x4 Ub[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        f32x4 acc = R[b];
#pragma unroll
        for (int m = 0; m < b; ++m)
          acc = mfma16(frag16(sL + 16 * b * PT + 16 * m, PT, lane), Ub[m], acc);
        const f32x4 u = mfma16(frag16(sm.tb + 16 * b * P16, P16, lane), pack16(acc), zero4());
        Ub[b] = pack16(u);
      }
      // O = Qhat S + M U
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
#pragma unroll
        for (int m = 0; m <= rt; ++m)
          O[rt] = mfma16(frag16(sM + 16 * rt * PT + 16 * m, PT, lane), Ub[m], O[rt]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.o[(16 * rt + 4 * g4 + i) * BV + 16 * wave + c16] = EL::put(O[rt][i]);
      }
      // U columns -> [c][t] operand of Wtil^T U
#pragma unroll
      for (int b = 0; b < 4; ++b)
        *reinterpret_cast<s16x4*>(&ub[c16 * PT + 16 * b + 4 * g4]) = Ub[b];
    } else {
      for (int e = lane; e < 16 * PT; e += 64) ub[e] = EL::put(0.f);
      wave_lds_sync();
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        f32x4 acc = R[b];
        if (b > 0) MM::run(acc, sL + 16 * b * PT, PT, ub, PT, b >= 3 ? 64 : 32, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) xb[c16 * P16 + 4 * g4 + i] = EL::put(acc[i]);
        wave_lds_sync();
        f32x4 u = zero4();
        MM::run(u, sm.tb + b * 16 * P16, P16, xb, P16, 16, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) ub[c16 * PT + 16 * b + 4 * g4 + i] = EL::put(u[i]);
        wave_lds_sync();
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        MM::run(O[rt], sM + 16 * rt * PT, PT, ub, PT, rt >= 2 ? 64 : 32, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sm.o[(16 * rt + 4 * g4 + i) * BV + 16 * wave + c16] = EL::put(O[rt][i]);
      }
    }
    wave_lds_sync();
    // S = diag(g_n) S + Wtil^T U
    {
      constexpr int KT = CH / MmaK<E>::v;
      Frag fu[KT];
#pragma unroll
      for (int s = 0; s < KT; ++s) fu[s] = MM::frag(ub, PT, lane, s);
      const float gsc = CHANNEL ? 1.f : sm.gam[CH - 1];
#pragma unroll
      for (int dt = 0; dt < DK / 16; ++dt) {
        Frag fw[KT];
#pragma unroll
        for (int s = 0; s < KT; ++s) fw[s] = MM::frag(sm.wt + 16 * dt * PT, PT, lane, s);
        if constexpr (CHANNEL) {
          const f32x4 gn = *reinterpret_cast<const f32x4*>(&sm.gn[16 * dt + 4 * g4]);
          S[dt] = S[dt] * gn;
        } else {
          S[dt] = S[dt] * gsc;
        }
#pragma unroll
        for (int s = 0; s < KT; ++s) S[dt] = MM::mma(fw[s], fu[s], S[dt]);
      }
    }
    __syncthreads();  // (F) output tile complete; chunk operands free

  }
  // the last chunk's output tile
  if (nchunks > 0) {
    const int cl = nchunks - 1;
    store_out(cl * CH, min(CH, T - cl * CH));
  }

  // ---- final state and auxiliary state (neither for a head flagged out of
  // range: the tokenwise pass writes them from S0 and aux0 as they are)
  const bool oor = CHANNEL && sm.oor;
  if (CHANNEL && a.oor && slice == 0 && tid == 0) a.oor[bh] = oor ? 1 : 0;
  float* const fin = xfer ? a.S_final_x : a.S_final;
  if (fin && !oor) {
    // transfer slices: their columns of S_final_x [B, H, dk, xcols]
    const int sstride = xfer ? a.xcols : a.dv;
    const int col = col0 + 16 * wave + c16 - (xfer ? a.dv : 0);
#pragma unroll
    for (int dt = 0; dt < DK / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 16 * dt + 4 * g4 + i;
        fin[(static_cast<long>(bh) * DK + row) * sstride + col] = S[dt][i];
      }
  }
  if (oor) return;
  if constexpr (PG2) {
    if (a.aux_final && slice == 0 && tid < DK)
      a.aux_final[static_cast<long>(bh) * DK + tid] = nchunks > 0 ? sm.acarry[tid] : aux[0];
  } else if (GAIN == GAIN_KDN_ISO) {
    if (a.aux_final && slice == 0 && tid == 0)
      a.aux_final[bh] = nchunks > 0 ? sm.acarry[0] : (a.aux0 ? a.aux0[bh] : 1.f);
  } else if ((GAIN == GAIN_PGDN || GAIN == GAIN_KDN) && a.aux_final && slice == 0) {
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      const int d = tid + cc * NT;
      if (d < DK) a.aux_final[static_cast<long>(bh) * DK + d] = aux[cc];
    }
  }
}

template <typename E, int DK, int BV, int GAIN, bool CHANNEL>
static hipError_t launch_one(const ChunkArgs& a, hipStream_t st) {
  constexpr bool HAS_W = CHANNEL || GAIN == GAIN_PGDN || GAIN == GAIN_KDN || GAIN == GAIN_EXPLICIT;
  using Sm = ChunkSmem<E, DK, BV, HAS_W>;
  auto kern = chunk_fwd_kernel<E, DK, BV, GAIN, CHANNEL>;
  const size_t smem = sizeof(Sm);
  static_assert(sizeof(Sm) <= 160 * 1024, "LDS budget");
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(smem));
  if (err != hipSuccess) return err;
  dim3 grid(static_cast<unsigned>(((a.dv + a.xcols) / BV) * a.B * a.H));
  hipLaunchKernelGGL(kern, grid, dim3(BV * 4), smem, st, a);
  return hipGetLastError();
}

template <typename E, int DK, int BV>
static hipError_t launch_gain(const ChunkArgs& a, int gain, bool channel, hipStream_t st) {
  if (channel) {
    switch (gain) {
      case GAIN_KLA: return launch_one<E, DK, BV, GAIN_KLA, true>(a, st);
      case GAIN_GDN: return launch_one<E, DK, BV, GAIN_GDN, true>(a, st);
      case GAIN_PGDN: return launch_one<E, DK, BV, GAIN_PGDN, true>(a, st);
      case GAIN_KDN: return launch_one<E, DK, BV, GAIN_KDN, true>(a, st);
      case GAIN_KDN_ISO: return launch_one<E, DK, BV, GAIN_KDN_ISO, true>(a, st);
      default: return launch_one<E, DK, BV, GAIN_EXPLICIT, true>(a, st);
    }
  }
  switch (gain) {
    case GAIN_KLA: return launch_one<E, DK, BV, GAIN_KLA, false>(a, st);
    case GAIN_GDN: return launch_one<E, DK, BV, GAIN_GDN, false>(a, st);
    case GAIN_PGDN: return launch_one<E, DK, BV, GAIN_PGDN, false>(a, st);
    case GAIN_KDN: return launch_one<E, DK, BV, GAIN_KDN, false>(a, st);
    case GAIN_KDN_ISO: return launch_one<E, DK, BV, GAIN_KDN_ISO, false>(a, st);
    default: return launch_one<E, DK, BV, GAIN_EXPLICIT, false>(a, st);
  }
}

hipError_t launch_chunk_fwd(const ChunkArgs& a, int io_bf16, int gain, bool channel,
                            hipStream_t st) {
  if (io_bf16) {
    if (!channel && gain != GAIN_KDN && gain != GAIN_KDN_ISO) return launch_chunk_fwd_bf16_scalar(a, gain, st);
    if (channel && gain != GAIN_PGDN) return launch_chunk_fwd_bf16_channel(a, gain, st);
    if (a.dk == 128) return launch_gain<uint16_t, 128, 64>(a, gain, channel, st);
    return launch_gain<uint16_t, 64, 64>(a, gain, channel, st);
  }
  if (a.dk == 64) return launch_gain<float, 64, 32>(a, gain, channel, st);
  return hipErrorInvalidValue;
}

}  // namespace dn
