// Chunked forward, bf16 operands: scalar decay (KLA, GDN, PGDN, explicit
// write vectors) and per-channel decay with the KDN gains (diagonal and
// isotropic): consumer, producer and loader wavefronts.
//
// Chunk form (our statement of Kaczmarz Linear Attention §2.5 Eqs. 7-9 and
// Preconditioned DeltaNet §2.6 Eq. 6), per chunk of 64 tokens with G the
// in-chunk cumulative log2-decay, g = 2^G and c_j the column scale (beta_j
// for KLA / GDN, whose write vector is c_j k_j; 1 where w is stored):
//   L = strict_lower(K W^T) 2^(G_i - G_j) c_j,  M = lower(Q W^T) 2^(G_i - G_j) c_j,
//   (I + L) U = V - diag(g) K S,   O = diag(g) Q S + M U,
//   S_out = g_n S + W^T diag(f) U,   f_j = 2^(G_n - G_j) c_j.
// With per-channel decay the operands carry the decay instead: K^, Q^ and W^
// are scaled per channel relative to token 31 (see cd_pass2) and S enters
// the products scaled by the decay from the chunk start to token 31.
//
// A workgroup owns one (batch, head) and 64 value columns and runs twelve
// wavefronts, three per SIMD:
//   consumers (waves 0..3): wave ct owns value columns 16 ct .. 16 ct + 15 and
//     keeps the whole d_k x 16 slice of S in registers.  Per chunk it forms
//     K S and (Q S)^T, runs the blocked triangular solve, adds M U, writes the
//     output tile and updates S.
//   producers (waves 4..7): build the chunk-local operands: the gains and
//     decays, the L and M tiles (the diagonal blocks and some of the twelve
//     off-diagonal tiles), the inverses of the diagonal blocks of I + L.
//   loaders (waves 8..11): issue every global load, one chunk step ahead,
//     stage it into LDS, and take the off-diagonal tiles and the share of the
//     statistic scans that their other work leaves room for.
// Scalar-decay gains formed from the staging registers (KLA, GDN, explicit):
// per chunk c, three phases separated by workgroup barriers:
//   P1  consumers: K S -> R = V - g K S, and (Q S)^T of c.
//       producers: the decay of c + 1; the off-diagonal L and M tiles of c
//       scaled; (I + L_bb)^-1 of c.  loaders: k, q of c + 1 into LDS, the
//       loads of k and the gates of c + 2; their off-diagonal tiles of c scaled.
//   P2  consumers: solve -> U; O = g Q S + M U -> HBM.
//       producers: the raw L and M tile products of c + 1 and its column
//       scales (the key norms of KLA are the diagonal of the raw K K^T).
//       loaders: v of c + 1 into LDS, the loads of q, v of c + 2; their raw
//       off-diagonal tiles of c + 1.
//   P3  consumers: S = g_n S + W^T diag(f) U.  producers: the diagonal L and
//       M blocks of c + 1 scaled.  loaders: the gates of c + 2 into LDS.
// PGDN, whose write vectors come out of a statistic scan over the LDS copy
// of k, forms its tiles of c in P1 and scans chunk c + 1 in P2 (pass 1) and
// P3 (pass 2) on producers and loaders.  The KDN gains run four phases per
// chunk (see the KDN loop).  Every load has a whole chunk step to arrive.  k,
// q, w and the gains are double buffered by chunk parity; every other LDS
// buffer is single: it is rewritten only after its last reader of the
// previous chunk has passed a barrier.
//
// Register-resident operands.  In v_mfma_f32_16x16x32_bf16 lane l supplies
// k = 8 (l / 16) .. +7 of its row (A) or column (B), and the accumulator holds
// rows 4 (l / 16) + i of column l % 16.  The contraction of one MFMA may use
// any pairing of k slots that A and B share, so a pair of packed accumulator
// tiles is the operand of one k-block as it stands, and the other operand is
// read in the matching order: the state tiles hold their key channels in the
// order of the 16-byte fragments of K and Q (see KLay), W^T comes from
// transposing ds_read_b64_tr_b16 reads, and M is stored with its token columns
// in the order of the packed U tiles (see mcol).  With 16x16x16 operands the
// accumulator layout already is the B layout (used by the solve).
#include "common.hpp"
#include "gains.hpp"
#include "launch.hpp"

namespace dn {

namespace ws {

constexpr int CH = 64;  // chunk length
constexpr int BV = 64;  // value columns per workgroup

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// DPP lane moves within rows of 16 lanes (gfx9 encodings: row_shr:n = 0x110 + n,
// row_bcast:15 = 0x142, row_bcast:31 = 0x143, quad_perm = 2-bit lane
// selectors).  Lanes masked off, or whose source lies outside the row, return
// `old`.
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ float dpp(float x, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(x), CTRL,
                                                    ROW_MASK, BANK_MASK, false));
}
// inclusive prefix sum over the 64 lanes of a wavefront
__device__ __forceinline__ float wave_prefix_sum(float x) {
  float s = x + dpp<0x111>(x, 0.f);
  s += dpp<0x112>(x, 0.f);
  s += dpp<0x113>(x, 0.f);
  s += dpp<0x114, 0xF, 0xE>(s, 0.f);
  s += dpp<0x118, 0xF, 0xC>(s, 0.f);
  s += dpp<0x142, 0xA, 0xF>(s, 0.f);
  s += dpp<0x143, 0xC, 0xF>(s, 0.f);
  return s;
}
// sum over each group of 4 consecutive lanes, in every lane of the group
__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<0xB1>(x, 0.f);  // quad_perm(1,0,3,2)
  x += dpp<0x4E>(x, 0.f);  // quad_perm(2,3,0,1)
  return x;
}
// sum over each group of N = 8 or 16 consecutive lanes (N | 16), in every lane
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x = quad_sum(x);
  x += dpp<0x141>(x, 0.f);  // row_half_mirror: the other quad of the 8
  if constexpr (N == 16) x += dpp<0x140>(x, 0.f);  // row_mirror: the other 8 of the 16
  return x;
}

// Raw buffer resource (stride 0, 32-bit data format) over nbytes from base:
// loads at offsets >= nbytes return 0 and stores there are dropped, which
// zero-fills the rows of a partial chunk and masks its output rows.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), nbytes,
                                           0x00020000);
}

// ---- MFMA operands
typedef short s16x4_lds __attribute__((ext_vector_type(4), address_space(3)));

__device__ __forceinline__ bf16x8 cat8(s16x4 lo, s16x4 hi) {
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  const u32x4 v = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(bf16x8, v);
}
// Transposing read (ds_read_b64_tr_b16): within each group of 16 lanes, lane
// l receives element l % 4 of the 8-byte chunk addressed by lane 4 j + l / 4,
// j = 0..3.  With lane (g, l) addressing row r0 + 4 g + l / 4, column
// c0 + 4 (l % 4) of a row-major matrix X, lane (g, l) receives X[r0 + 4 g + j]
// [c0 + l], j = 0..3: four consecutive rows of one column.
__device__ __forceinline__ s16x4 read_tr(const uint16_t* p, int ld, int lane, int r0, int c0) {
  const uint16_t* a = p + (r0 + 4 * (lane >> 4) + ((lane & 15) >> 2)) * ld + c0 + 4 * (lane & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_lds*)(a));
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ s16x4 frag16(const uint16_t* p, int ld, int lane) {
  return __builtin_bit_cast(
      s16x4, *reinterpret_cast<const u32x2*>(p + (lane & 15) * ld + 4 * (lane >> 4)));
}
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ s16x4 pack16(f32x4 c) {
  const u32x2 v = {pack_bf2(c[0], c[1]), pack_bf2(c[2], c[3])};
  return __builtin_bit_cast(s16x4, v);
}
__device__ __forceinline__ f32x4 unpack16(s16x4 p) {
  const u32x2 v = __builtin_bit_cast(u32x2, p);
  return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xFFFF0000u),
               __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xFFFF0000u)};
}

// Layout of the [token][d_k] tiles k, q, w in LDS: row-major rows of
// d_k + 16 bf16.  Measured on gfx950, the 16-byte fragment reads of 16 rows
// by 4 lane groups are free of bank conflicts at this pitch (the 8-byte
// half reads are not), and every fragment address is one per-lane base plus a
// compile-time offset.
//
// State tile rows.  A consumer's packed state operand of k-block s (the
// accumulator tiles 2 s and 2 s + 1, rows 4 g + i) must meet one 16-byte
// fragment of K or Q, i.e. key channels 32 s + 8 g .. +7.  So row 4 g + i of
// state tile 2 s + h holds key channel 32 s + 8 g + 4 h + i; the update's
// transposing reads of W^T fetch those channels (sigma_channel).
template <int DK>
struct KLay {
  static constexpr int P = DK + 16;
  static __device__ __forceinline__ int idx(int r, int d) { return r * P + d; }
  // per-lane base of the fragment reads: row lane % 16, k-group lane / 16
  static __device__ __forceinline__ int frag_base(int lane) { return (lane & 15) * P + 8 * (lane >> 4); }
  // row0 + lane % 16 (row0 a multiple of 16), k = 32 s + 8 (lane / 16) .. +7
  static __device__ __forceinline__ bf16x8 frag32(const uint16_t* b, int fb, int row0, int s) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(b + fb + row0 * P + 32 * s));
  }
  // per-lane base of the transposing reads: addressing lane a = 4 j + q of
  // group g reads row 4 g + j, channel group 8 q
  static __device__ __forceinline__ int tr_base(int lane) {
    const int a = lane & 15;
    return (4 * (lane >> 4) + (a >> 2)) * P + 8 * (a & 3);
  }
  // A operand of W^T for state tile 2 s + h over tokens r0 + 4 g + j (r0 a
  // multiple of 16): lane (g, l) receives W[r0 + 4 g + j][sigma(l)], j = 0..3,
  // sigma(l) = 32 s + 8 (l / 4) + 4 h + l % 4 (see read_tr); tb = tr_base(lane)
  static __device__ __forceinline__ s16x4 read_tr(const uint16_t* b, int tb, int r0, int s, int h) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_lds*)(b + tb + r0 * P + 32 * s + 4 * h));
  }
  // four consecutive tokens r0 .. r0 + 3 of channel cb + lane as fp32, one
  // transposing read: lane 4 j + q of group g addresses token r0 + j,
  // channels cb + 16 g + 4 q .. +3, so every lane receives its own channel
  static __device__ __forceinline__ f32x4 col4(const uint16_t* b, int r0, int cb, int lane) {
    const int a = lane & 15;
    const uint16_t* p = b + (r0 + (a >> 2)) * P + cb + 16 * (lane >> 4) + 4 * (a & 3);
    return unpack16(__builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4_lds*)p));
  }
  // key channel of row 4 g + i of state tile dt
  static __device__ __forceinline__ int sigma_channel(int dt, int g, int i) {
    return 32 * (dt >> 1) + 8 * g + 4 * (dt & 1) + i;
  }
};

// Column order of the M tiles in LDS: within each block of 32 tokens, token
// group (4 tokens) gr sits at position 2 (gr mod 4) + gr / 4, so that M U
// reads the token pairs {32 s + 4 g .. +3, 32 s + 16 + 4 g .. +3} that the
// packed U tiles hold as one 16-byte piece at 32 s + 8 g.
__device__ __forceinline__ int mcol(int j) {
  const int gr = (j >> 2) & 7;
  return (j & ~31) + 4 * (2 * (gr & 3) + (gr >> 2)) + (j & 3);
}

// wavefront roles: 0 consumer, 1 producer, 2 loader
template <int R>
struct Role {
  static constexpr int role = R;
};
// Twelve wavefronts, three per SIMD: loaders (waves 8..11) issue every load
// and stage it into LDS, so that no consumer or producer ever waits on the
// memory pipeline (which backs up when all CUs ask for their next chunk at
// once).  Per chunk c the loaders stage k, q of c + 1 (PGDN: and its gates) and
// load k and the gates of c + 2 in P1, stage v of c + 1 and load q, v of c + 2
// in P2, and (the other gains) stage the gates of c + 2 in P3.
constexpr int WS_THREADS = 768;

template <int DK, int GAIN>
struct Smem {
  static constexpr int PK = KLay<DK>::P;  // [token][d_k] rows, bf16 (see KLay)
  static constexpr int PV = BV + 16;  // [token][value] rows, bf16
  static constexpr int PT = CH + 8;   // [token][token] rows, bf16
  static constexpr int P16 = 16 + 8;  // rows of 16-wide blocks
  static constexpr bool HAS_W = GAIN == GAIN_PGDN || GAIN == GAIN_EXPLICIT;
  // per-channel decay: diagonal and isotropic KDN, and KLA / GDN / explicit w
  // (GAIN_*_CD)
  static constexpr bool CD = GAIN == GAIN_KDN || GAIN == GAIN_KDN_ISO || GAIN >= GAIN_CD;
  static constexpr bool PG = GAIN == GAIN_PGDN;
  // KDN: k holds raw k, then (in place) the scaled write vectors W^, by parity;
  // q[0] raw q, then Q^ in place; q[1] K^; w[0], w[1] the raw alpha, omega
  alignas(16) uint16_t k[2][CH * PK];           // k, by chunk parity
  alignas(16) uint16_t w[HAS_W || CD ? 2 : 1][HAS_W || CD ? CH * PK : 8];  // write vectors, by parity
  alignas(16) uint16_t q[2][CH * PK];           // q, by chunk parity
  alignas(16) uint16_t v[CH * PV];              // value slice
  alignas(16) uint16_t ln[CH * PT];             // -L [i][j], the off-diagonal 16x16 tiles
  alignas(16) uint16_t mp[CH * PT];             // M [i][j]
  alignas(16) uint16_t tb[4 * 16 * P16];        // (I + L_bb)^-1 [r][c], blocks b = 0..3
  alignas(16) float g2[2][CH];                  // cumulative log2-decay, by chunk parity
  alignas(16) float gam[2][CH];                 // 2^g2, by chunk parity
  alignas(16) float cs[2][CH];                  // column scale c_j, by chunk parity
  alignas(16) float kap[2][CH];                 // 2^(E_b(j) - G_j) c_j, E_b = G at the end of j's block
  alignas(16) float fs[CH];                     // S-update scale f_j
  alignas(16) float galpha[2][CH];              // staged alpha, eta by chunk parity (loaders)
  alignas(16) float geta[2][CH];
  alignas(16) float eta[PG ? CH : 4];           // per-token gates (PGDN)
  alignas(16) float alpha[PG ? CH : 4];
  alignas(16) float ap[PG ? CH : 4];
  alignas(16) float bp[PG ? CH : 4];
  alignas(16) float ah[PG ? 512 : 4];           // PGDN: statistic at the segment ends [seg][d_k]
  alignas(16) float acarry[DK];                 // PGDN / KDN: statistic / variance carried between chunks
  float segp[8];                                // PGDN: product of alphaP over each segment
  // KDN: per [segment][d_k] the variance map of the segment (m00, m01, m10,
  // m11) and its decay product; per d_k and chunk parity the decay to the
  // reference token and from it to the chunk end
  alignas(16) float msum[CD ? 5 : 1][CD ? 512 : 4];
  alignas(16) float gref[CD ? 2 : 1][CD ? DK : 4];
  alignas(16) float gnr[CD ? 2 : 1][CD ? DK : 4];
  int oor;  // per-channel decay: some chunk was beyond the range of the chunk form
};

// OUT = false: an instance for launches without an output (a.o == NULL): the
// consumers leave out Q S and M U, the producers and loaders the M tiles, and
// q is not read.
template <int DK, int GAIN, bool OUT>
__device__ __forceinline__ void chunk_fwd_ws_body(const ChunkArgs& a) {
  constexpr int NT = WS_THREADS;        // threads
  constexpr int NP = 256;               // producer threads
  constexpr int NDT = DK / 16;          // state tiles of a consumer
  constexpr int KS = DK / 32;           // k-blocks of a d_k contraction
  constexpr int VEC = 8;                // bf16 per 16-byte access
  constexpr int KV_LOADS = CH * DK / (NP * VEC);  // 16-byte pieces of k (q, w) per producer
  constexpr int V_LOADS = CH * BV / (NP * VEC);
  constexpr bool HAS_W = GAIN == GAIN_PGDN || GAIN == GAIN_EXPLICIT;
  constexpr bool PG = GAIN == GAIN_PGDN;
  // Per-channel decay (CD): diagonal KDN (a variance per channel), isotropic
  // KDN (one variance per head, Kalman Delta Networks §2.7, Eq. 40), and KLA,
  // GDN (KDA) and explicit w (CDX), which have no variance: their write
  // vectors are the keys (or w) scaled like isotropic KDN's, their column
  // scales the gain's.  All share the decay-scaled operands of this mode.
  constexpr bool CDX = GAIN >= GAIN_CD;
  constexpr int BG = CDX ? GAIN - GAIN_CD : GAIN;  // the write gain of a CDX instance
  constexpr bool CD = GAIN == GAIN_KDN || GAIN == GAIN_KDN_ISO || CDX;
  constexpr bool ISO = GAIN == GAIN_KDN_ISO;
  constexpr bool KD = GAIN == GAIN_KDN;    // a variance per key channel
  constexpr bool NOVAR = ISO || CDX;       // no per-channel variance scan
  constexpr bool HAS_ETA = GAIN != GAIN_EXPLICIT && !CD;
  // Gains straight from the staging registers (no per-channel scan): the
  // gains of chunk c + 1 are formed in P2 as it is staged, and its tiles in
  // P3.  PGDN scans its statistic over the LDS copy of k in P3 and forms its
  // tiles in P1, once its write vectors exist.
  constexpr bool REG = !PG && !CD;
  using Sm = Smem<DK, GAIN>;
  constexpr int PV = Sm::PV, PT = Sm::PT, P16 = Sm::P16;
  using KL = KLay<DK>;
  static_assert(KV_LOADS * NP * VEC == CH * DK && V_LOADS * NP * VEC == CH * BV, "tile split");
  static_assert(NP % DK == 0 && CH % (2 * NP / DK) == 0 && (CH / (2 * NP / DK)) % 4 == 0 && 2 * NP / DK <= 8,
                "statistic scan layout");

  extern __shared__ __align__(16) unsigned char smem_raw[];
  DN_LDS_POISON(smem_raw, sizeof(Sm));
  Sm& sm = *reinterpret_cast<Sm*>(smem_raw);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g4 = lane >> 4, c16 = lane & 15;

  // XCD-aware mapping of the 1-D grid: consecutive workgroups are dealt to the
  // 8 XCDs in turn, so the value slices of one head get ids that are equal
  // modulo 8 and share that XCD's L2 (k and q come from HBM once).
  const int ns = (a.dv + a.xcols) / BV;  // value slices (and transfer slices)
  const int nwg = ns * a.B * a.H;
  int bh, slice;
  {
    const int id = blockIdx.x;
    if (nwg % 8 == 0 && (nwg / 8) % ns == 0) {
      const int xcd = id % 8, r = id / 8;
      slice = r % ns;
      bh = xcd * (nwg / 8 / ns) + r / ns;
    } else {
      slice = id % ns;
      bh = id / ns;
    }
  }
  const int h = bh % a.H;
  const int col0 = slice * BV;
  // a transfer slice: columns col0 - dv of S0 = I, v = 0, no output
  const bool xfer = col0 >= a.dv;
  const int T = a.T;
  const int nchunks = (T + CH - 1) / CH;
  const long qk_base = static_cast<long>(bh) * T * DK;
  const long v_base = static_cast<long>(bh) * T * a.dv;

  // the M tiles above the diagonal that M U reads with its 32-token k-blocks
  // (rows 0..15 x tokens 16..31, rows 32..47 x tokens 48..63) are zeros
  for (int e = tid; e < 2 * 256; e += NT) {
    const int bi = 2 * (e >> 8), r = (e >> 4) & 15, x = e & 15;
    sm.mp[(16 * bi + r) * PT + mcol(16 * (bi + 1) + x)] = 0;
  }

  auto run = [&](auto role) __attribute__((always_inline)) {
    constexpr int RO = decltype(role)::role;
    constexpr bool CONS = RO == 0, PROD = RO == 1, LOAD = RO == 2;
    const int ct = wave;           // consumers: column tile
    const int pw = wave - 4;       // producers: wavefront index
    const int ptid = tid - 256;    // producers: thread index
    // the role's own thread index (its share of the staging)
    const int ltid = tid - 256 * RO;
    const int fb = KL::frag_base(lane), trb = KL::tr_base(lane);  // LDS operand bases

    // consumers: byte offsets of the output pieces (token 16 rt + c16, value
    // columns col0 + 16 ct + 4 g4 .. +3) inside a chunk
    int ooff[4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) ooff[rt] = 2 * ((16 * rt + c16) * a.dv + col0 + 16 * ct + 4 * g4);

    // ---------------- consumer state: element i of tile dt = key channel
    // sigma_channel(dt, g4, i), value column c16 of the wave's 16
    f32x4 S[CONS ? NDT : 1];
    const int sstride = xfer ? a.xcols : a.dv, scol0 = xfer ? col0 - a.dv : col0;
    const long s_lane = (static_cast<long>(bh) * DK + 8 * g4) * sstride + scol0 + 16 * ct + c16;
    if constexpr (CONS) {
      if (xfer) {
        // S0 = I: the state after a segment is then its transfer matrix
        const int col = scol0 + 16 * ct + c16;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) S[dt][i] = KL::sigma_channel(dt, g4, i) == col ? 1.f : 0.f;
      } else if (a.S0) {
        const float* base = a.S0 + s_lane;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) S[dt][i] = base[(KL::sigma_channel(dt, 0, i)) * a.dv];
      } else {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) S[dt] = zero4();
      }
    } else if constexpr (PROD) {
      if ((PG || KD) && ptid < DK) sm.acarry[ptid] = a.aux0 ? a.aux0[static_cast<long>(bh) * DK + ptid] : 1.f;
      // isotropic KDN: the head's variance entering chunk x sits in acarry[x % 2]
      if (ISO && ptid == 0) sm.acarry[0] = a.aux0 ? a.aux0[bh] : 1.f;
      if (CD && ptid == 0) sm.oor = 0;
      // KDN: the decay lives in the operands, the token-decay arrays stay 0 / 1
      if (CD && ptid < 2 * CH) {
        sm.g2[ptid >> 6][ptid & 63] = 0.f;
        sm.gam[ptid >> 6][ptid & 63] = 1.f;
      }
    }

    // ---------------- producer staging of one chunk: 16-byte pieces, rows
    // of k / q / w in consecutive lanes (coalesced), likewise for v
    u32x4 pk[KV_LOADS], pq[KV_LOADS], pwv[GAIN == GAIN_EXPLICIT ? KV_LOADS : 1], pv[V_LOADS];
    u32x4 pa[CD ? KV_LOADS : 1], po[CD ? KV_LOADS : 1];  // KDN: alpha, omega pieces
    float l_alpha = 1.f, l_eta = 0.f, l_ap = 1.f, l_bp = 0.f;  // loaders: gates of token ltid
    float l_om = 0.f;  // loaders: isotropic KDN process noise of token ltid
    float pg_start = 0.f;  // PGDN: carried statistic read by pass 1 (segment 0)

    // per-lane byte offsets inside a chunk: the k / q / w pieces (row-major
    // [CH][DK]) and the value pieces (row t, columns col0 + cc of [T][dv])
    int koff[KV_LOADS], voff[V_LOADS];
#pragma unroll
    for (int j = 0; j < KV_LOADS; ++j) koff[j] = 2 * (ltid + j * NP) * VEC;
#pragma unroll
    for (int j = 0; j < V_LOADS; ++j) {
      const int e = (ltid + j * NP) * VEC;
      voff[j] = 2 * ((e / BV) * a.dv + col0 + e % BV);
    }
    // tokens of chunk c (0 past the end).  The clamp lowers to a vector
    // v_med3; read back as a scalar, the buffer resources built from it stay
    // in scalar registers (else every load becomes a readfirstlane loop)
    auto ntok = [&](int c) __attribute__((always_inline)) {
      return __builtin_amdgcn_readfirstlane(max(0, min(CH, T - c * CH)));
    };
    // loads of chunk c through buffer resources that end at its last token:
    // past the end k = q = w = v = eta = alphaP = betaP = 0 (alpha, alphaP are
    // replaced by 1 where they are used).  Chunks past the last one get empty
    // resources, so the loads ahead are issued unconditionally: a load under a
    // branch leaves a register merge after it that waits for the load.
    // k (w, gates) and q, v are loaded, and staged, at different points
    auto fetch_k = [&](int c) __attribute__((always_inline)) {
      const int t0 = c * CH;
      const int n = ntok(c);
      const long tok = static_cast<long>(bh) * T + t0;
      const auto rk = rsrc(static_cast<const uint16_t*>(a.k) + qk_base + static_cast<long>(t0) * DK, 2 * n * DK);
#pragma unroll
      for (int j = 0; j < KV_LOADS; ++j) {
        pk[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff[j], 0, 0);
        if constexpr (GAIN == GAIN_EXPLICIT) {
          const auto rw = rsrc(static_cast<const uint16_t*>(a.g.w) + qk_base + static_cast<long>(t0) * DK, 2 * n * DK);
          pwv[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, koff[j], 0, 0);
        }
      }
    };
    auto fetch_q = [&](int c) __attribute__((always_inline)) {
      const int t0 = c * CH;
      const int n = ntok(c);
      // without an output q is not needed: an empty resource, every load returns 0
      const auto rq = OUT ? rsrc(static_cast<const uint16_t*>(a.q) + qk_base + static_cast<long>(t0) * DK, 2 * n * DK)
                          : rsrc(a.k, 0);
#pragma unroll
      for (int j = 0; j < KV_LOADS; ++j) pq[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, koff[j], 0, 0);
    };
    // KDN: the per-channel alpha and omega of chunk c (laid out like k)
    auto fetch_ao = [&](int c) __attribute__((always_inline)) {
      if constexpr (CD) {
        const int t0 = c * CH;
        const int n = ntok(c);
        const long off = qk_base + static_cast<long>(t0) * DK;
        const auto ra = rsrc(static_cast<const uint16_t*>(a.g.alpha) + off, 2 * n * DK);
#pragma unroll
        for (int j = 0; j < KV_LOADS; ++j) pa[j] = __builtin_amdgcn_raw_buffer_load_b128(ra, koff[j], 0, 0);
        // diagonal KDN: omega; explicit w: w (isotropic KDN's omega is a
        // per-token scalar, with the gates)
        if constexpr (KD || (CDX && BG == GAIN_EXPLICIT)) {
          const auto rw = rsrc(static_cast<const uint16_t*>(KD ? a.g.omega : a.g.w) + off, 2 * n * DK);
#pragma unroll
          for (int j = 0; j < KV_LOADS; ++j) po[j] = __builtin_amdgcn_raw_buffer_load_b128(rw, koff[j], 0, 0);
        }
      }
    };
    auto fetch_v = [&](int c) __attribute__((always_inline)) {
      const int t0 = c * CH;
      const int n = ntok(c);
      // v == NULL: an empty resource, every load returns 0
      const auto rv = a.v && !xfer
                          ? rsrc(static_cast<const uint16_t*>(a.v) + v_base + static_cast<long>(t0) * a.dv, 2 * n * a.dv)
                          : rsrc(a.k, 0);
#pragma unroll
      for (int j = 0; j < V_LOADS; ++j) pv[j] = __builtin_amdgcn_raw_buffer_load_b128(rv, voff[j], 0, 0);
    };
    // registers -> LDS for chunk c of n tokens (the loads already hold zeros
    // past the end; alpha = alphaP = 1 there)
    auto stash_q = [&](int c) __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < KV_LOADS; ++j) {
        const int e = (ltid + j * NP) * VEC;
        *reinterpret_cast<u32x4*>(&sm.q[CD ? 0 : c & 1][KL::idx(e / DK, e % DK)]) = pq[j];
      }
    };
    // KDN: alpha, omega of a chunk of n tokens into LDS; alpha past the end
    // is 1 (omega, k and the information scale are 0 there), so the variance
    // and the decay pass through the padding unchanged
    auto stash_ao = [&](int n) __attribute__((always_inline)) {
      if constexpr (CD) {
#pragma unroll
        for (int j = 0; j < KV_LOADS; ++j) {
          const int e = (ltid + j * NP) * VEC;
          const int t = e / DK, d = e % DK;
          const u32x4 one = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
          *reinterpret_cast<u32x4*>(&sm.w[0][KL::idx(t, d)]) = t < n ? pa[j] : one;
          if constexpr (KD || (CDX && BG == GAIN_EXPLICIT))
            *reinterpret_cast<u32x4*>(&sm.w[1][KL::idx(t, d)]) = po[j];
          if constexpr (ISO || (CDX && BG == GAIN_KLA)) {
            // ||k_t||^2 (isotropic KDN, KLA) and the sum of alpha_t^2 over the
            // channels (isotropic KDN), from the staging registers (DK / 8
            // consecutive lanes per token; k is 0 and alpha 1 past the end)
            const u32x4 al4 = t < n ? pa[j] : one;
            float sk = 0.f, sa = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float k0 = __uint_as_float(pk[j][i] << 16), k1 = __uint_as_float(pk[j][i] & 0xFFFF0000u);
              sk = fmaf(k0, k0, fmaf(k1, k1, sk));
              if constexpr (ISO) {
                const float a0 = __uint_as_float(al4[i] << 16), a1 = __uint_as_float(al4[i] & 0xFFFF0000u);
                sa = fmaf(a0, a0, fmaf(a1, a1, sa));
              }
            }
            sk = group_sum<DK / VEC>(sk);
            if constexpr (ISO) sa = group_sum<DK / VEC>(sa);
            if (d == 0) {
              sm.msum[4][t] = sk;
              if constexpr (ISO) sm.msum[4][CH + t] = sa;
            }
          }
        }
      }
    };
    auto stash_v = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int j = 0; j < V_LOADS; ++j) {
        const int e = (ltid + j * NP) * VEC;
        *reinterpret_cast<u32x4*>(&sm.v[(e / BV) * PV + e % BV]) = pv[j];
      }
    };
    auto stash_k = [&](int c, int n) __attribute__((always_inline)) {
      uint16_t* kb = sm.k[c & 1];
#pragma unroll
      for (int j = 0; j < KV_LOADS; ++j) {
        const int e = (ltid + j * NP) * VEC;
        const int t = e / DK, d = e % DK;
        *reinterpret_cast<u32x4*>(&kb[KL::idx(t, d)]) = pk[j];
        if constexpr (GAIN == GAIN_EXPLICIT) *reinterpret_cast<u32x4*>(&sm.w[c & 1][KL::idx(t, d)]) = pwv[j];
      }
    };

    // ---------------- loaders: per-token gates of chunk c (the first
    // loader wavefront, token = lane) into registers, then into LDS
    auto fetch_gates = [&](int c) __attribute__((always_inline)) {
      const int t0 = c * CH;
      const int n = ntok(c);
      const long tok = static_cast<long>(bh) * T + t0;
      if constexpr (CDX) {
        // KLA / GDN: eta_t (alpha is per channel, in its own tile)
        if constexpr (BG != GAIN_EXPLICIT)
          l_eta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(a.g.eta + tok, 4 * n), 4 * ltid, 0, 0));
        return;
      } else if constexpr (CD) {
        // KDN: the observation noise r_t (alpha is per channel, in its own tile);
        // isotropic KDN also its process noise omega_t
        l_eta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(a.g.r + tok, 4 * n), 4 * ltid, 0, 0));
        if constexpr (ISO)
          l_om = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              rsrc(static_cast<const float*>(a.g.omega) + tok, 4 * n), 4 * ltid, 0, 0));
        return;
      }
      l_alpha = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(rsrc(static_cast<const float*>(a.g.alpha) + tok, 4 * n), 4 * ltid, 0, 0));
      if constexpr (HAS_ETA)
        l_eta = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(a.g.eta + tok, 4 * n), 4 * ltid, 0, 0));
      if constexpr (PG) {
        l_ap = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(a.g.alphaP + tok, 4 * n), 4 * ltid, 0, 0));
        l_bp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc(a.g.betaP + tok, 4 * n), 4 * ltid, 0, 0));
      }
    };
    // REG: alpha, eta by chunk parity; PGDN: the per-token gate arrays of the
    // statistic scan (alpha, alphaP past the end of n tokens are 1)
    auto stash_gates = [&](int c, int n) __attribute__((always_inline)) {
      if (ltid < CH) {
        if constexpr (CD) {
          // r_t, and the information scale mu / r_t of the variance update
          // (0 past the end)
          sm.geta[c & 1][ltid] = l_eta;
          // isotropic KDN: omega_t instead (0 past the end); KLA / GDN: eta_t
          // in geta, nothing here
          sm.galpha[c & 1][ltid] = ISO ? l_om : KD && ltid < n ? a.g.mu_info * __builtin_amdgcn_rcpf(l_eta) : 0.f;
        } else if constexpr (PG) {
          const bool ok = ltid < n;
          sm.eta[ltid] = l_eta;
          sm.alpha[ltid] = ok ? l_alpha : 1.f;
          sm.ap[ltid] = ok ? l_ap : 1.f;
          sm.bp[ltid] = l_bp;
        } else {
          sm.galpha[c & 1][ltid] = l_alpha;
          sm.geta[c & 1][ltid] = l_eta;
        }
      }
    };

    // ---------------- producers (REG): cumulative decay of chunk c of n tokens
    // (wavefront 0, token = lane; alpha past the end counts as 1)
    auto regains = [&](int c, int n) __attribute__((always_inline)) {
      if (pw == 0) {
        const float x = wave_prefix_sum(log2_hw(lane < n ? sm.galpha[c & 1][lane] : 1.f));
        sm.g2[c & 1][lane] = x;
        sm.gam[c & 1][lane] = exp2_hw(x);
      }
    };
    // ---------------- producers: gains of a staged chunk c of n tokens from
    // its LDS copy (PGDN)
    // part 1: cumulative decay and column scales (producers), PGDN statistic
    // pass 1 (producers and loaders: scan thread sid of 2 NP)
    constexpr int NSEG = 2 * NP / DK, SL = CH / NSEG;  // PGDN scan segments of SL tokens
    const int sid = CONS ? 0 : (PROD ? ptid : NP + ltid);
    auto gains1 = [&](int c) __attribute__((always_inline)) {
      const uint16_t* kb = sm.k[c & 1];
      if constexpr (PROD) {
        if (pw == 0) {
          const float x = wave_prefix_sum(log2_hw(sm.alpha[lane]));
          sm.g2[c & 1][lane] = x;
          sm.gam[c & 1][lane] = exp2_hw(x);
          // kap_t = 2^(E_b - G_t), E_b = G at the end of t's block of 16
          sm.kap[c & 1][lane] = exp2_hw(__shfl(x, lane | 15) - x);
        }
        if (ptid < CH) sm.cs[c & 1][ptid] = 1.f;
      }
      if constexpr (PG) {
        // the statistic scan in NSEG segments of the chunk: pass 1 runs
        // each segment from 0 (segment 0 from the carried statistic)
        const int d = sid % DK, g = sid / DK, cb = d & ~63;  // the wavefront's 64 channels
        pg_start = g == 0 ? sm.acarry[d] : 0.f;
        float st = pg_start, pr = 1.f;
#pragma unroll
        for (int t4 = 0; t4 < SL; t4 += 4) {
          const int t = g * SL + t4;
          const f32x4 kk = KL::col4(kb, t, cb, lane);
          const f32x4 ap4 = *reinterpret_cast<const f32x4*>(&sm.ap[t]);
          const f32x4 bp4 = *reinterpret_cast<const f32x4*>(&sm.bp[t]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            st = pgdn_stat(st, ap4[j], bp4[j], kk[j]);
            pr *= ap4[j];
          }
        }
        sm.ah[g * DK + d] = st;
        if (d == 0) sm.segp[g] = pr;
      }
    };
    // part 2 (PGDN, after a barrier): the exact start of segment g is
    // E_(g-1), E_0 = end of segment 0, E_g = P_g E_(g-1) + (pass-1 end of g);
    // each segment is replayed from it and writes its w = eta B(A) k
    auto gains2 = [&](int c) __attribute__((always_inline)) {
      if constexpr (PG) {
        const int d = sid % DK, g = sid / DK;
        const uint16_t* kb = sm.k[c & 1];
        uint16_t* wb = sm.w[c & 1];
        float At = pg_start;
        if (g > 0) {
          At = sm.ah[d];
          for (int gg = 1; gg < g; ++gg) At = fmaf(sm.segp[gg], At, sm.ah[gg * DK + d]);
        }
        // the write scale B(A) = exp(-ln(x) s), s = r / (1 + |r|), r = ln A - mu
        // (Preconditioned DeltaNet §2.4, Eq. 9) on the hardware log2 / rcp /
        // exp2: B = 2^(y / (1 + |r|)) with y = -log2(x) r one fma of log2 A,
        // and 1 + |r| = 1 + |y| / log2(x)
        const float l2x = a.g.log2x;
        const float cy = -l2x * 0.69314718055994531f, y0 = l2x * a.g.mu_log[h];
        const float il2x = __builtin_amdgcn_rcpf(l2x);
        const int cb = d & ~63;
#pragma unroll
        for (int t4 = 0; t4 < SL; t4 += 4) {
          const int t = g * SL + t4;
          const f32x4 kk = KL::col4(kb, t, cb, lane);
          const f32x4 ap4 = *reinterpret_cast<const f32x4*>(&sm.ap[t]);
          const f32x4 bp4 = *reinterpret_cast<const f32x4*>(&sm.bp[t]);
          const f32x4 et4 = *reinterpret_cast<const f32x4*>(&sm.eta[t]);
          // two tokens per conversion; the halves go to their two rows
#pragma unroll
          for (int j = 0; j < 4; j += 2) {
            float xw[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              At = pgdn_stat(At, ap4[j + h2], bp4[j + h2], kk[j + h2]);
              const float y = fmaf(log2_hw(At), cy, y0);
              const float bs = exp2_hw(y * __builtin_amdgcn_rcpf(fmaf(fabsf(y), il2x, 1.0f)));
              xw[h2] = et4[j + h2] * bs * kk[j + h2];
            }
            const uint32_t pw2 = pack_bf2(xw[0], xw[1]);
            wb[KL::idx(t + j, d)] = static_cast<uint16_t>(pw2);
            wb[KL::idx(t + j + 1, d)] = static_cast<uint16_t>(pw2 >> 16);
          }
        }
        // the carried statistic is read again only by the next chunk's pass 1
        if (g == NSEG - 1) sm.acarry[d] = At;
      }
    };

    // ---------------- KDN (per-channel decay): the variance scan of a staged
    // chunk c in NSEG segments of SL tokens per key channel (scan thread sid:
    // channel sid % DK, segment sid / DK; producers and loaders).  One token
    // maps the variance p to p_hat / (1 + u p_hat), p_hat = alpha^2 p + omega,
    // u = (mu / r) k^2 (Kalman Delta Networks §2.4-2.5): the Mobius map with
    // coefficients (alpha^2, omega; u alpha^2, 1 + u omega), and a segment's
    // updates compose to one such map.  Pass 1 composes each segment's map and
    // its decay product; pass 2 starts each segment from the carried variance
    // through the maps of the segments before it, replays its tokens and
    // writes the decay-scaled operands of the chunk form,
    //   K^ = k 2^(G_t - G_r),  Q^ = q 2^(G_t - G_r),  W^ = p_hat k 2^(G_r - G_t),
    // G_t the log-decay from the chunk start through token t (per channel) and
    // G_r its value at token 31.  The gain's column scale 1 / (r + z) comes
    // later from the diagonal of K^ W^T (z_t = sum of p_hat k^2).
    float cd_p0 = 1.f;  // the carried variance, read in pass 1 (pass 2 of the
                        // last segment rewrites the carry)
    auto cd_pass1 = [&](int c) __attribute__((always_inline)) {
      if constexpr (CD) {
        const int d = sid % DK, g = sid / DK, cb = d & ~63;
        const uint16_t* kb = sm.k[c & 1];
        if constexpr (KD) cd_p0 = sm.acarry[d];
        float m00 = 1.f, m01 = 0.f, m10 = 0.f, m11 = 1.f, pr = 1.f;
#pragma unroll 1
        for (int t4 = 0; t4 < SL; t4 += 4) {
          const int t = g * SL + t4;
          const f32x4 al = KL::col4(sm.w[0], t, cb, lane);
          if constexpr (NOVAR) {  // no variance per channel: the segment's decay product only
            pr *= al[0] * al[1] * (al[2] * al[3]);
            continue;
          }
          const f32x4 kk = KL::col4(kb, t, cb, lane);
          const f32x4 om = KL::col4(sm.w[1], t, cb, lane);
          const f32x4 mu4 = *reinterpret_cast<const f32x4*>(&sm.galpha[c & 1][t]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // M_t = [[1, 0], [u, 1]] [[a^2, omega], [0, 1]]: the prediction
            // acts on the top row, the update adds u times it to the bottom row
            const float aa = al[j] * al[j];
            const float u = mu4[j] * kk[j] * kk[j];
            m00 = fmaf(aa, m00, om[j] * m10);
            m01 = fmaf(aa, m01, om[j] * m11);
            m10 = fmaf(u, m00, m10);
            m11 = fmaf(u, m01, m11);
            pr *= al[j];
          }
          // the map is projective: divide by its (1, 1) entry, which is >= 1
          const float sc = __builtin_amdgcn_rcpf(m11);
          m00 *= sc;
          m01 *= sc;
          m10 *= sc;
          m11 = 1.f;
        }
        sm.msum[0][sid] = m00;
        sm.msum[1][sid] = m01;
        sm.msum[2][sid] = m10;
        sm.msum[3][sid] = pr;
      }
    };
    auto cd_pass2 = [&](int c) __attribute__((always_inline)) {
      if constexpr (CD) {
        const int d = sid % DK, g = sid / DK, cb = d & ~63;
        constexpr int RS = NSEG / 2 - 1;  // the segment that ends at token 31
        float p = cd_p0, num = 1.f, den = 1.f, gr = 1.f, gt = 1.f;
#pragma unroll
        for (int gg = 0; gg < NSEG; ++gg) {
          const float pr = sm.msum[3][gg * DK + d];
          if (gg < g) {
            if constexpr (KD)
              p = fmaf(sm.msum[0][gg * DK + d], p, sm.msum[1][gg * DK + d]) *
                  __builtin_amdgcn_rcpf(fmaf(sm.msum[2][gg * DK + d], p, 1.f));
            if (gg > RS) num *= pr;
          } else if (gg <= RS) {
            den *= pr;
          }
          if (gg <= RS) gr *= pr;
          else gt *= pr;
        }
        // 2^(G - G_r) before the segment's first token
        float e = num * __builtin_amdgcn_rcpf(den);
        if (g == 0) {
          // 2^(G_r): chunk start -> token 31; 2^(G_n - G_r): token 31 -> chunk
          // end.  Referred to token 31, every factor stays within 2^96 and S
          // 2^(G_r) stays normal while both half-chunk decays are at least
          // 2^-96; beyond that the chunk form cannot be evaluated this way, and
          // a NaN reference turns the head's state and every later output
          // into NaN rather than into wrong finite values
          const bool in_range = gr >= 0x1p-96f && gt >= 0x1p-96f;
          sm.gref[c & 1][d] = in_range ? gr : __builtin_nanf("");
          sm.gnr[c & 1][d] = gt;
          if (!in_range) sm.oor = 1;  // the head is recomputed token by token
        }
        uint16_t* kw = sm.k[c & 1];  // raw k, rewritten in place with W^
        uint16_t* qh = sm.q[0];      // raw q, rewritten in place with Q^
        uint16_t* kh = sm.q[1];      // K^
#pragma unroll 1
        for (int t4 = 0; t4 < SL; t4 += 4) {
          const int t = g * SL + t4;
          const f32x4 kk = KL::col4(kw, t, cb, lane);
          const f32x4 qq = OUT ? KL::col4(qh, t, cb, lane) : zero4();
          const f32x4 al = KL::col4(sm.w[0], t, cb, lane);
          // diagonal KDN: omega; explicit w: w
          const f32x4 om = KD || BG == GAIN_EXPLICIT ? KL::col4(sm.w[1], t, cb, lane) : zero4();
          const f32x4 mu4 = KD ? *reinterpret_cast<const f32x4*>(&sm.galpha[c & 1][t]) : zero4();
          // the decay 2^(G_t - G_r) at the four tokens, and its inverse: one
          // reciprocal at the last token, then back through the alphas
          f32x4 et, ie;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            e *= al[j];
            et[j] = e;
          }
          ie[3] = __builtin_amdgcn_rcpf(e);
#pragma unroll
          for (int j = 3; j > 0; --j) ie[j - 1] = ie[j] * al[j];
          // two tokens per step: one conversion packs the pair, whose halves
          // go to their two rows
#pragma unroll
          for (int j = 0; j < 4; j += 2) {
            float xk[2], xq[2], xw[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const int jj = j + h2;
              xk[h2] = kk[jj] * et[jj];
              xq[h2] = qq[jj] * et[jj];
              if constexpr (NOVAR) {
                // isotropic KDN, KLA, GDN: W^ = k 2^(G_r - G_t) (explicit: w in
                // place of k); the gain (beta_t, eta_t / (||k_t||^2 + eps),
                // eta_t, 1) is the column scale
                xw[h2] = (BG == GAIN_EXPLICIT ? om[jj] : kk[jj]) * ie[jj];
              } else {
                const float ph = fmaf(al[jj] * al[jj], p, om[jj]);
                const float pk = ph * kk[jj];
                xw[h2] = pk * ie[jj];
                // p_hat / (1 + u p_hat) with u p_hat = (mu / r) k (p_hat k)
                p = ph * __builtin_amdgcn_rcpf(fmaf(mu4[jj] * kk[jj], pk, 1.f));
              }
            }
            const uint32_t pkh = pack_bf2(xk[0], xk[1]), pqh = pack_bf2(xq[0], xq[1]),
                           pkw = pack_bf2(xw[0], xw[1]);
            kh[KL::idx(t + j, d)] = static_cast<uint16_t>(pkh);
            kh[KL::idx(t + j + 1, d)] = static_cast<uint16_t>(pkh >> 16);
            if constexpr (OUT) {
              qh[KL::idx(t + j, d)] = static_cast<uint16_t>(pqh);
              qh[KL::idx(t + j + 1, d)] = static_cast<uint16_t>(pqh >> 16);
            }
            kw[KL::idx(t + j, d)] = static_cast<uint16_t>(pkw);
            kw[KL::idx(t + j + 1, d)] = static_cast<uint16_t>(pkw >> 16);
          }
        }
        if (KD && g == NSEG - 1) sm.acarry[d] = p;
      }
    };

    // LDS operands of chunk c: keys, queries and write vectors (KDN: the
    // decay-scaled K^, Q^ and W^)
    auto opk = [&](int c) __attribute__((always_inline)) -> const uint16_t* {
      return CD ? sm.q[1] : sm.k[c & 1];
    };
    auto opq = [&](int c) __attribute__((always_inline)) -> const uint16_t* {
      return CD ? sm.q[0] : sm.q[c & 1];
    };
    auto opw = [&](int c) __attribute__((always_inline)) -> const uint16_t* {
      return CD ? sm.k[c & 1] : HAS_W ? sm.w[c & 1] : sm.k[c & 1];
    };

    // ---------------- producers and loaders: tile products of chunk c (raw,
    // in registers).  Producer p owns the diagonal block p (L_pp in both
    // orientations, M_pp) and items 3 p .. 3 p + NIT_P - 1 of the twelve
    // off-diagonal tiles (L or M of (bi, bj), bj < bi), loader l items
    // 3 l + NIT_P .. 3 l + 2: the loaders take what their other work (PGDN's
    // statistic scan) leaves room for.  Item it is of kind
    // it % 2 (0: L, 1: M)
    // and covers tile (bi, bj) = pair it / 2 of (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
    auto item_is_m = [](int it) { return (it & 1) != 0; };
    auto item_bi = [](int it) { const int pr = it >> 1; return pr < 1 ? 1 : pr < 3 ? 2 : 3; };
    auto item_bj = [](int it) { const int pr = it >> 1; return pr < 1 ? 0 : pr < 3 ? pr - 1 : pr - 3; };
    // Items per producer: REG, GDN and explicit w with per-channel decay 1,
    // PGDN 2, the KDN modes and KLA with per-channel decay 3; the loaders take
    // the rest (those with key norms or a variance scan to form take none)
    constexpr int NIT_P = PG ? 2 : KD || ISO || (CDX && BG == GAIN_KLA) ? 3 : 1;
    constexpr int NIT = LOAD ? 3 - NIT_P : NIT_P;  // off-diagonal items of this wavefront
    const int lw = wave - 8;  // loaders: wavefront index
    auto item_of = [&](int k) { return PROD ? 3 * pw + k : 3 * lw + NIT_P + k; };  // wave-uniform
    f32x4 at = zero4(), an = zero4(), mt = zero4(), off[NIT > 0 ? NIT : 1];
#pragma unroll
    for (int k = 0; k < NIT; ++k) off[k] = zero4();
    auto tiles = [&](int c) __attribute__((always_inline)) {
      const uint16_t* kb = opk(c);
      const uint16_t* qb = opq(c);
      const uint16_t* wb = opw(c);
      const int p = pw;
      at = an = mt = zero4();
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kp = KL::frag32(kb, fb, 16 * p, s);
        bf16x8 qp;
        if constexpr (OUT) qp = KL::frag32(qb, fb, 16 * p, s);  // M only with an output
        const bf16x8 wp = HAS_W || CD ? KL::frag32(wb, fb, 16 * p, s) : kp;
        at = mfma32(wp, kp, at);  // lane: [j = 16p + 4 g4 + u][i = 16p + c16]
        if constexpr (OUT) mt = mfma32(wp, qp, mt);
        an = mfma32(kp, wp, an);  // lane: [i = 16p + 4 g4 + u][j = 16p + c16]
      }
    };
    auto tiles_off = [&](int c) __attribute__((always_inline)) {
      const uint16_t* kb = opk(c);
      const uint16_t* qb = opq(c);
      const uint16_t* wb = opw(c);
#pragma unroll
      for (int k = 0; k < NIT; ++k) {
        const int it = item_of(k);
        if (!OUT && item_is_m(it)) continue;  // M tiles only with an output
        const int bi = item_bi(it), bj = item_bj(it);
        const uint16_t* xsrc = item_is_m(it) ? qb : kb;
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < KS; ++s)
          acc = mfma32(KL::frag32(wb, fb, 16 * bj, s), KL::frag32(xsrc, fb, 16 * bi, s), acc);
        off[k] = acc;
      }
    };

    // ---------------- producers (REG): the column scales of chunk c, set by
    // the lane of each token t = 16 p + (lane % 16) that holds the diagonal
    // entry w_t . k_t of the raw product at (for KLA ||k_t||^2, exact: bf16
    // products are exact in fp32); also kap_t = 2^(E_p - G_t) c_t
    // KDN: the column scales of the diagonal block in registers, for
    // scale_diag in the same phase: cdi for token 16 p + c16 (the lane's row of
    // an), cdj for tokens 16 p + 4 g4 + u (its columns of at and mt)
    float cdi = 0.f;
    f32x4 cdj = zero4();
    auto diag_gains = [&](int c, int n) __attribute__((always_inline)) {
      if constexpr (ISO) {
        // isotropic KDN (Kalman Delta Networks §2.7, Eq. 40), lane = token t of
        // the chunk: the head's variance runs through the chunk as a prefix
        // product of the Moebius maps b -> (a b + omega) / (u a b + 1 + u omega),
        // u = mu ||k||^2 / (d_k r), a = mean alpha^2 (padding: the identity).
        // Every producer wavefront forms the same scan, so each has the step
        // sizes beta_t = b_hat / (r + b_hat ||k||^2) of its block in registers.
        const int t = lane;
        const bool ok = t < n;
        const float nk = sm.msum[4][t], am = sm.msum[4][CH + t] * (1.0f / DK);
        const float om = sm.galpha[c & 1][t], rr = ok ? sm.geta[c & 1][t] : 1.f;
        const float u = ok ? a.g.mu_info * nk / (DK * rr) : 0.f;
        float m00 = am, m01 = om, m10 = u * am, m11 = fmaf(u, om, 1.f);
        // inclusive scan by DPP lane moves: shifts by 1, 2, 4, 8 within rows
        // of 16 lanes, then row 0's and row 2's last lane into rows 1 and 3,
        // and lane 31 into rows 2 and 3.  A lane with no source receives the
        // identity map, so every lane composes at every step:
        // (maps of its own span) o (maps before)
        auto compose = [&](float y00, float y01, float y10, float y11) __attribute__((always_inline)) {
          const float n00 = fmaf(m00, y00, m01 * y10), n01 = fmaf(m00, y01, m01 * y11);
          const float n10 = fmaf(m10, y00, m11 * y10), n11 = fmaf(m10, y01, m11 * y11);
          const float sc = __builtin_amdgcn_rcpf(n11);  // projective: keep (1, 1) at 1
          m00 = n00 * sc;
          m01 = n01 * sc;
          m10 = n10 * sc;
          m11 = 1.f;
        };
#define DN_ISO_STEP(CTRL, RM)                                                                  \
  compose(dpp<CTRL, RM>(m00, 1.f), dpp<CTRL, RM>(m01, 0.f), dpp<CTRL, RM>(m10, 0.f),          \
          dpp<CTRL, RM>(m11, 1.f))
        DN_ISO_STEP(0x111, 0xF);
        DN_ISO_STEP(0x112, 0xF);
        DN_ISO_STEP(0x114, 0xF);
        DN_ISO_STEP(0x118, 0xF);
        DN_ISO_STEP(0x142, 0xA);
        DN_ISO_STEP(0x143, 0xC);
#undef DN_ISO_STEP
        const float b0 = sm.acarry[c & 1];
        // variance after token t (hardware reciprocals, as in the other gains)
        const float bt = fmaf(m00, b0, m01) * __builtin_amdgcn_rcpf(fmaf(m10, b0, m11));
        // the variance before token t: lane t - 1's, b0 in lane 0 (DPP wave_shr:1)
        const float bp = dpp<0x138>(bt, b0);
        const float bh_ = fmaf(am, bp, om);
        const float beta = ok ? bh_ * __builtin_amdgcn_rcpf(fmaf(bh_, nk, rr)) : 0.f;
        if (pw == 0 && lane == CH - 1) sm.acarry[(c + 1) & 1] = bt;
        cdi = __shfl(beta, 16 * pw + c16);
#pragma unroll
        for (int u4 = 0; u4 < 4; ++u4) cdj[u4] = __shfl(beta, 16 * pw + 4 * g4 + u4);
      } else if constexpr (CDX) {
        // KLA, GDN, explicit w: the column scale of token t is the gain's,
        // eta_t / (||k_t||^2 + eps) with the raw keys' norm (Kaczmarz Linear
        // Attention §2.1), eta_t, or 1; 0 past the end
        auto colscale = [&](int t) __attribute__((always_inline)) {
          const float g = BG == GAIN_KLA   ? sm.geta[c & 1][t] * __builtin_amdgcn_rcpf(sm.msum[4][t] + a.g.eps)
                        : BG == GAIN_GDN   ? sm.geta[c & 1][t]
                                           : 1.f;
          return t < n ? g : 0.f;
        };
        cdi = colscale(16 * pw + c16);
#pragma unroll
        for (int u = 0; u < 4; ++u) cdj[u] = colscale(16 * pw + 4 * g4 + u);
      } else if constexpr (KD) {
        // the diagonal entry z_t of token t = 16 p + x sits in lane 16 (x / 4) + x,
        // slot x % 4; the other lanes of the block fetch it with a lane shuffle
        const float zs = c16 & 2 ? (c16 & 1 ? at[3] : at[2]) : (c16 & 1 ? at[1] : at[0]);
        const float* rr = sm.geta[c & 1] + 16 * pw;
        const float zi = __shfl(zs, 16 * (c16 >> 2) + c16);
        cdi = 16 * pw + c16 < n ? __builtin_amdgcn_rcpf(rr[c16] + zi) : 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float zj = __shfl(zs, 20 * g4 + u);
          cdj[u] = 16 * pw + 4 * g4 + u < n ? __builtin_amdgcn_rcpf(rr[4 * g4 + u] + zj) : 0.f;
        }
      }
      if (g4 == (c16 >> 2)) {
        const int u = c16 & 3, t = 16 * pw + c16;
        const float nk = u == 0 ? at[0] : u == 1 ? at[1] : u == 2 ? at[2] : at[3];
        // KLA step size eta / (||k||^2 + eps) (Kaczmarz Linear Attention §2.1),
        // with the hardware reciprocal; GDN: eta; stored write vectors: 1
        const float et = sm.geta[c & 1][t];
        // KDN: nk = K^_t . W^_t = z_t, the sum of p_hat k^2 over the channels,
        // and the gain's column scale is 1 / (r_t + z_t) (Kalman Delta
        // Networks §2.4)
        float cv = GAIN == GAIN_KLA ? et * __builtin_amdgcn_rcpf(nk + a.g.eps)
                 : GAIN == GAIN_GDN ? et
                 : CD ? cdi : 1.f;
        cv = t < n ? cv : 0.f;
        sm.cs[c & 1][t] = cv;
        sm.kap[c & 1][t] = CD ? cv : cv * exp2_hw(sm.g2[c & 1][16 * pw + 15] - sm.g2[c & 1][t]);
      }
    };

    // ---------------- producers: scale the raw tile products with the gains
    // in LDS (2^(G_i - G_j) c_j, masks), store M_pp and the off-diagonal -L
    // and M tiles; at, an keep the scaled L_pp for the inverse.  Off the
    // diagonal (j in block bj < bi) the factor is 2^(G_i - E_bj) kap_j with
    // E_bj = G at the end of block bj: both factors are at most c_j, so
    // neither overflows however strong the decay
    // diagonal block (scale_diag) and off-diagonal tiles (scale_off): the
    // inverse needs the first, the consumers' solve and M U the second
    auto scale_diag = [&](int c) __attribute__((always_inline)) {
      const int p = pw;
      const float* g2 = sm.g2[c & 1];
      const float* cs = sm.cs[c & 1];
      // (KDN: the scales come from diag_gains' registers; the LDS copy is
      // written in this same phase by other lanes)
      const float gd_i = CD ? 0.f : g2[16 * p + c16], cd_i = CD ? 0.f : cs[16 * p + c16];
      const f32x4 gd_j = CD ? zero4() : *reinterpret_cast<const f32x4*>(&g2[16 * p + 4 * g4]);
      const f32x4 cd_j = CD ? zero4() : *reinterpret_cast<const f32x4*>(&cs[16 * p + 4 * g4]);
      // diagonal block p: at = A^T (row i = 16p + c16, columns j = 16p + 4 g4 + u),
      // an = A (transposed roles), mt = M_pp like at
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float f = CD ? cdj[u] : exp2_hw(gd_i - gd_j[u]) * cd_j[u];
        at[u] = (4 * g4 + u < c16) ? at[u] * f : 0.f;
        mt[u] = (4 * g4 + u <= c16) ? mt[u] * f : 0.f;
        an[u] = (c16 < 4 * g4 + u) ? an[u] * (CD ? cdi : exp2_hw(gd_j[u] - gd_i) * cd_i) : 0.f;
      }
      if constexpr (OUT)
        *reinterpret_cast<u32x2*>(&sm.mp[(16 * p + c16) * PT + mcol(16 * p + 4 * g4)]) =
            u32x2{pack_bf2(mt[0], mt[1]), pack_bf2(mt[2], mt[3])};
    };
    auto scale_off = [&](int c) __attribute__((always_inline)) {
      const float* g2 = sm.g2[c & 1];
      float rho[NIT > 0 ? NIT : 1];
      f32x4 ko_j[NIT > 0 ? NIT : 1];
#pragma unroll
      for (int k = 0; k < NIT; ++k) {
        const int it = item_of(k);
        const float sg = item_is_m(it) ? 1.f : -1.f;
        rho[k] = CD ? sg : sg * exp2_hw(g2[16 * item_bi(it) + c16] - g2[16 * item_bj(it) + 15]);
        ko_j[k] = *reinterpret_cast<const f32x4*>(&sm.kap[c & 1][16 * item_bj(it) + 4 * g4]);
      }
#pragma unroll
      for (int k = 0; k < NIT; ++k) {
        const int it = item_of(k);
        const bool m = item_is_m(it);
        if (!OUT && m) continue;
        f32x4 val;
#pragma unroll
        for (int u = 0; u < 4; ++u) val[u] = off[k][u] * (rho[k] * ko_j[k][u]);
        const int jc = 16 * item_bj(it) + 4 * g4;
        uint16_t* dst = (m ? sm.mp : sm.ln) + (16 * item_bi(it) + c16) * PT + (m ? mcol(jc) : jc);
        *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf2(val[0], val[1]), pack_bf2(val[2], val[3])};
      }
    };
    // ---------------- producers: (I + L_pp)^-1 from at = acc(A^T), an = acc(A),
    // A = L_pp strictly lower: (I + A)^-1 = (I - A)(I + A^2)(I + A^4)(I + A^8);
    // and the S-update scale f_j = 2^(G_n - G_j) c_j.  Packed, an accumulator
    // tile acc(X) is the A operand of X^T and the B operand of X, so one
    // 16x16x16 MFMA gives C + X^T Y.  The powers and partial products enter as
    // bf16 (fp32 accumulation), the rounding the stored inverse gets anyway;
    // (I + Z)^T Y = Y + Z^T Y: each identity term is the exact fp32 start value
    // of the accumulator
    const int ud = c16 - 4 * g4;  // the slot of this lane's diagonal entry, if 0..3
    const f32x4 idm = {ud == 0 ? 1.f : 0.f, ud == 1 ? 1.f : 0.f, ud == 2 ? 1.f : 0.f, ud == 3 ? 1.f : 0.f};
    auto invert = [&](int c) __attribute__((always_inline)) {
      if (pw == 1)
        sm.fs[lane] = CD ? sm.cs[c & 1][lane] : sm.cs[c & 1][lane] * exp2_hw(sm.g2[c & 1][CH - 1] - sm.g2[c & 1][lane]);
      const s16x4 sat = pack16(at), san = pack16(an);
      const f32x4 A2 = mfma16(sat, san, zero4()), A2t = mfma16(san, sat, zero4());
      const s16x4 sA2 = pack16(A2), sA2t = pack16(A2t);
      const f32x4 A4 = mfma16(sA2t, sA2, zero4()), A4t = mfma16(sA2, sA2t, zero4());
      const s16x4 sA4 = pack16(A4), sA4t = pack16(A4t);
      const f32x4 A8 = mfma16(sA4t, sA4, zero4());
      const f32x4 imt = idm - at;                               // (I - A)^T
      const f32x4 p1t = mfma16(sA2, pack16(imt), imt);          // ((I - A)(I + A^2))^T
      const f32x4 p2t = mfma16(sA4, pack16(p1t), p1t);          // ... (I + A^4)
      const f32x4 tt_ = mfma16(pack16(A8), pack16(p2t), p2t);   // acc(T^T)
      // lane holds T[c16][4 g4 + u]: row c16 of block p
      *reinterpret_cast<u32x2*>(&sm.tb[(16 * pw + c16) * P16 + 4 * g4]) =
          u32x2{pack_bf2(tt_[0], tt_[1]), pack_bf2(tt_[2], tt_[3])};
    };

    // ---------------- consumers, per chunk c (bodies of the three phases)
    f32x4 R[4], OQ[4];
    float gn = 1.f;         // g_n of chunk c (gam is rewritten in P2 / P3)
    bf16x8 U0, U1, F0, F1;  // U and diag(f) U, k-blocks 0 and 1 (tiles 0,1 and 2,3)
    // the backward's checkpoints (no-output instances with S_ck / E_ck): one
    // byte offset per lane, the row or key channel in the resource base or the
    // scalar offset, so that no address register is rewritten between stores
    const int ek_voff = 4 * (4 * g4 * a.dv + col0 + 16 * ct + c16);  // E: row 4 g4 of the resource
    const int ck_voff = 4 * (8 * g4 * a.dv + col0 + 16 * ct + c16);  // S_ck: channel 8 g4 + sigma(dt, 0, i)
    // S, the state entering chunk cidx, to S_ck
    auto store_ck = [&](int cidx) __attribute__((always_inline)) {
      if constexpr (CONS && !OUT && !CD) {
        const auto rs = rsrc(a.S_ck + (static_cast<long>(bh) * nchunks + cidx) * DK * a.dv, 4 * DK * a.dv);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[dt][i]), rs, ck_voff,
                                                  4 * KL::sigma_channel(dt, 0, i) * a.dv, 0);
      }
    };
    // P1: K S -> R = V - g K S, and (Q S)^T.  KDN: S is scaled per key channel
    // by 2^(G_r) first (the operands carry the decay relative to token 31)
    auto cons_p1 = [&](int c) __attribute__((always_inline)) {
      if constexpr (CONS) {
        const uint16_t* kb = opk(c);
        const uint16_t* qb = opq(c);
        // packed state: k-block s = tiles 2 s and 2 s + 1
        if constexpr (CD) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            S[dt] = S[dt] * *reinterpret_cast<const f32x4*>(&sm.gref[c & 1][KL::sigma_channel(dt, g4, 0)]);
        }
        bf16x8 Spk[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) Spk[s] = cat8(pack16(S[2 * s]), pack16(S[2 * s + 1]));
        // the value tiles and decays of all four row tiles are read first: LDS
        // reads complete in order, so a wait for one read issued after the
        // next row tile's fragments would also wait for those fragments
        s16x4 vt[4];
        f32x4 gt[4];
        float go[4];
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          vt[rt] = read_tr(sm.v, PV, lane, 16 * rt, 16 * ct);
          gt[rt] = *reinterpret_cast<const f32x4*>(&sm.gam[c & 1][16 * rt + 4 * g4]);
          go[rt] = sm.gam[c & 1][16 * rt + c16];
        }
        // K and Q fragments of row tile rt + 1 are read while rt multiplies
        bf16x8 kf[KS], qf[OUT ? KS : 1];
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          kf[s] = KL::frag32(kb, fb, 0, s);
          if constexpr (OUT) qf[s] = KL::frag32(qb, fb, 0, s);
        }
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          bf16x8 kn[KS], qn[OUT ? KS : 1];
          if (rt < 3) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
              kn[s] = KL::frag32(kb, fb, 16 * (rt + 1), s);
              if constexpr (OUT) qn[s] = KL::frag32(qb, fb, 16 * (rt + 1), s);
            }
          }
          f32x4 ak = zero4(), aq = zero4();
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            ak = mfma32(kf[s], Spk[s], ak);
            if constexpr (OUT) aq = mfma32(Spk[s], qf[s], aq);
          }
          if (rt < 3) {
#pragma unroll
            for (int s = 0; s < KS; ++s) {
              kf[s] = kn[s];
              if constexpr (OUT) qf[s] = qn[s];
            }
          }
          // R[t][c] = V[t][c] - g_t (K S)[t][c], rows t = 16 rt + 4 g4 + i
          const f32x4 vv = unpack16(vt[rt]);
          R[rt] = CD ? vv - ak : vv - gt[rt] * ak;
          // (Q S)^T[c][t] scaled by g_t, token t = 16 rt + c16
          if constexpr (OUT) OQ[rt] = CD ? aq : aq * go[rt];
        }
        gn = sm.gam[c & 1][CH - 1];
      }
    };
    // P2: solve -> U; O = g Q S + M U -> HBM
    auto cons_p2 = [&](int c, int t0, int n) __attribute__((always_inline)) {
      if constexpr (CONS) {
        // U_b = (I + L_bb)^-1 (R_b - sum_{m<b} L_bm U_m); every operand of the
        // chain is read up front (in the order it is used)
        s16x4 Ub[4], Fb[4], lt[6], tv[4];
        f32x4 fv[4];
        f32x4 Ek[!OUT && !CD ? 4 : 1];  // the residuals, kept for the checkpoint stores
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
          for (int m = 0; m < b; ++m) lt[b * (b - 1) / 2 + m] = frag16(sm.ln + 16 * b * PT + 16 * m, PT, lane);
          tv[b] = frag16(sm.tb + 16 * b * P16, P16, lane);
          fv[b] = *reinterpret_cast<const f32x4*>(&sm.fs[16 * b + 4 * g4]);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          f32x4 acc = R[b];
#pragma unroll
          for (int m = 0; m < b; ++m) acc = mfma16(lt[b * (b - 1) / 2 + m], Ub[m], acc);
          const f32x4 u = mfma16(tv[b], pack16(acc), zero4());
          Ub[b] = pack16(u);
          Fb[b] = pack16(u * fv[b]);
          if constexpr (!OUT && !CD) Ek[b] = u;
        }
        if constexpr (!OUT && !CD) {
          // the backward's residuals: E rows 16 b + 4 g4 + i of value column
          // col0 + 16 ct + c16, one lane offset for all (row 16 b + i in the
          // resource's base, rows past the end outside its range)
          if (a.E_ck) {
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int row = 16 * b + i;
                const auto re = rsrc(a.E_ck + v_base + static_cast<long>(t0 + row) * a.dv, 4 * max(0, n - row) * a.dv);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(Ek[b][i]), re, ek_voff, 0, 0);
              }
          }
        }
        U0 = cat8(Ub[0], Ub[1]);
        U1 = cat8(Ub[2], Ub[3]);
        F0 = cat8(Fb[0], Fb[1]);
        F1 = cat8(Fb[2], Fb[3]);
        if constexpr (OUT) {
          // O^T = g (Q S)^T + (M U)^T: lane holds value columns 16 ct + 4 g4 .. +3
          // of token 16 rt + c16; rows past the end fall outside the resource
          // a transfer slice: an empty resource, every store is dropped
          const auto ro = a.o && !xfer
                              ? rsrc(static_cast<uint16_t*>(a.o) + v_base + static_cast<long>(t0) * a.dv, 2 * n * a.dv)
                              : rsrc(a.k, 0);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt) {
            const uint16_t* mrow = sm.mp + (16 * rt + c16) * PT + 8 * g4;
            f32x4 o = mfma32(U0, __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(mrow)), OQ[rt]);
            if (rt >= 2) o = mfma32(U1, __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(mrow + 32)), o);
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3])}, ro,
                                                  ooff[rt], 0, 0);
          }
        }
        // PGDN: v of chunk c + 1 into LDS (chunk c's was last read in P1),
        // the loads of q and v of chunk c + 2 (the loads of k go out in P3)
      }
    };
    // P3: S = g_n S + W^T diag(f) U
    auto cons_p3 = [&](int c) __attribute__((always_inline)) {
      if constexpr (CONS) {
        const uint16_t* wb = opw(c);
        // S_dt = g_n S_dt + W^T diag(f) U: A = W^T read transposed from the
        // [token][d_k] rows of chunk c (tokens 32 s + 4 g4 + j and + 16)
        auto update = [&](int dt) __attribute__((always_inline)) {
          f32x4 acc = CD ? S[dt] : S[dt] * gn;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const bf16x8 wa = cat8(KL::read_tr(wb, trb, 32 * s, dt >> 1, dt & 1),
                                   KL::read_tr(wb, trb, 32 * s + 16, dt >> 1, dt & 1));
            acc = mfma32(wa, s == 0 ? F0 : F1, acc);
          }
          // KDN: S carries 2^(G_r) since P1; 2^(G_n - G_r) completes the decay
          S[dt] = CD ? acc * *reinterpret_cast<const f32x4*>(&sm.gnr[c & 1][KL::sigma_channel(dt, g4, 0)]) : acc;
        };
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) update(dt);
      }
    };

    if constexpr (CD) {
      // ---------------- KDN, per-channel decay: four phases per chunk c
      //   P1  consumers: K^ S, Q^ S of c.  producers: scale_off and the
      //       inverses of c.  loaders: k, alpha, omega, r of c + 1 into LDS,
      //       their loads for c + 2.
      //   P2  consumers: solve and output of c.  loaders: q, v of c + 1 into
      //       LDS.  producers and loaders: scan pass 1 of c + 1.
      //   P3  consumers: state update of c.  producers and loaders: scan
      //       pass 2 of c + 1 (writes K^, Q^, W^ of c + 1).
      //   P4  producers: the raw tile products of c + 1, its column scales
      //       from their diagonal, and its scaled diagonal blocks.  loaders:
      //       the loads of q, v of c + 2.
      if (nchunks > 0) {
        if constexpr (LOAD) {
          // (without an output nothing reads q or Q^: neither is formed)
          const int n0 = ntok(0);
          fetch_k(0);
          if constexpr (OUT) fetch_q(0);
          fetch_v(0);
          fetch_ao(0);
          fetch_gates(0);
          stash_k(0, n0);
          if constexpr (OUT) stash_q(0);
          stash_v();
          stash_ao(n0);
          stash_gates(0, n0);
          fetch_k(1);
          fetch_ao(1);
          fetch_gates(1);
          if constexpr (OUT) fetch_q(1);
          fetch_v(1);
        }
      }
      __syncthreads();
      if constexpr (!CONS) {
        if (nchunks > 0) cd_pass1(0);
      }
      __syncthreads();
      if constexpr (!CONS) {
        if (nchunks > 0) cd_pass2(0);
      }
      __syncthreads();
      if constexpr (PROD) {
        if (nchunks > 0) {
          tiles(0);
          tiles_off(0);
          diag_gains(0, ntok(0));
          scale_diag(0);
        }
      } else if constexpr (LOAD) {
        if (nchunks > 0) tiles_off(0);
      }
      __syncthreads();
      for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * CH;
        const int n = min(CH, T - t0);
        const int n1 = ntok(c + 1);
        // P1
        if constexpr (CONS) {
          cons_p1(c);
        } else if constexpr (LOAD) {
          if (c + 1 < nchunks) {
            stash_k(c + 1, n1);
            stash_ao(n1);
            stash_gates(c + 1, n1);
          }
          fetch_k(c + 2);
          fetch_ao(c + 2);
          fetch_gates(c + 2);
          scale_off(c);  // their off-diagonal tiles of chunk c
        } else {
          scale_off(c);
          invert(c);
        }
        __syncthreads();  // (1) L, M, (I + L_bb)^-1, f of chunk c ready
        // P2
        if constexpr (CONS) {
          cons_p2(c, t0, n);
        } else {
          if constexpr (LOAD) {
            if (c + 1 < nchunks) {
              if constexpr (OUT) stash_q(c + 1);
              stash_v();
            }
          }
          if (c + 1 < nchunks) cd_pass1(c + 1);
        }
        __syncthreads();  // (2) pass 1 of chunk c + 1 done; chunk c's solve done
        // P3
        if constexpr (CONS) {
          cons_p3(c);
        } else {
          if (c + 1 < nchunks) cd_pass2(c + 1);
        }
        __syncthreads();  // (3) K^, Q^, W^ of chunk c + 1 ready; S updated
        // P4
        if constexpr (PROD) {
          if (c + 1 < nchunks) {
            tiles(c + 1);
            tiles_off(c + 1);
            diag_gains(c + 1, n1);
            scale_diag(c + 1);
          }
        } else if constexpr (LOAD) {
          // the loads of q and v of chunk c + 2 (staged in P2 of chunk c + 1),
          // issued here, where the loaders have no scan work to hold back;
          // the raw products of their off-diagonal tiles of chunk c + 1
          if constexpr (OUT) fetch_q(c + 2);
          fetch_v(c + 2);
          if (c + 1 < nchunks) tiles_off(c + 1);
        }
        __syncthreads();  // (4) column scales and diagonal blocks of chunk c + 1 ready
      }
    } else {
      // ---------------- prologue: chunk 0 staged, its gains (and, REG, tiles)
      if (nchunks > 0) {
        // loaders: chunk 0 (REG: and the gates of chunk 1) into LDS; the loads
        // the loop stages first (k, q, v and, PGDN, the gates of chunk 1)
        // (without an output nothing reads q: it is neither loaded nor staged)
        if constexpr (LOAD) {
          fetch_k(0);
          if constexpr (OUT) fetch_q(0);
          fetch_v(0);
          fetch_gates(0);
          stash_k(0, min(CH, T));
          if constexpr (OUT) stash_q(0);
          stash_v();
          stash_gates(0, min(CH, T));
          fetch_gates(1);
          if constexpr (REG) stash_gates(1, ntok(1));
          fetch_k(1);
          if constexpr (OUT) fetch_q(1);
          fetch_v(1);
          // REG: q is staged two chunks ahead (in P3), so chunk 1's now
          if constexpr (REG && OUT) {
            if (nchunks > 1) stash_q(1);
          }
        }
      }
      __syncthreads();
      if constexpr (REG) {
        if (PROD && nchunks > 0) regains(0, min(CH, T));
        __syncthreads();
      }
      if (nchunks > 0) {
        if constexpr (REG) {
          if constexpr (PROD) {
            tiles(0);
            tiles_off(0);
            diag_gains(0, min(CH, T));
          } else if constexpr (LOAD) {
            tiles_off(0);
          }
        } else if constexpr (!CONS) {
          gains1(0);
        }
      }
      __syncthreads();
      if (nchunks > 0) {
        if constexpr (REG) {
          if constexpr (PROD) scale_diag(0);
        } else if constexpr (!CONS) {
          gains2(0);
        }
      }
      __syncthreads();

      for (int c = 0; c < nchunks; ++c) {
        const int t0 = c * CH;
        const int n = min(CH, T - t0);
        const int n1 = min(CH, T - t0 - CH);  // tokens of chunk c + 1 (if any)

        // ================= P1 =================
        if constexpr (CONS) {
          if (!OUT && a.S_ck && c == 0) store_ck(0);
          cons_p1(c);
        } else if constexpr (LOAD) {
          // k, q (PGDN: and the gates) of chunk c + 1 into LDS (REG: q goes in
          // P3, away from the consumers' fragment reads of this phase); the
          // loads of k and of the gates of chunk c + 2 (REG: and of q)
          if (c + 1 < nchunks) {
            stash_k(c + 1, n1);
            if constexpr (!REG && OUT) stash_q(c + 1);
            if constexpr (PG) stash_gates(c + 1, n1);
          }
          fetch_k(c + 2);
          fetch_gates(c + 2);
          if constexpr (REG && OUT) fetch_q(c + 2);
          // their off-diagonal tiles of chunk c (PGDN: the raw products too)
          if constexpr (PG) tiles_off(c);
          scale_off(c);
        } else {
          if constexpr (!REG) {
            tiles(c);
            tiles_off(c);
            scale_diag(c);
          }
          // REG: the decay of chunk c + 1 from its staged gates
          if constexpr (REG) {
            if (c + 1 < nchunks) regains(c + 1, n1);
          }
          scale_off(c);
          invert(c);
        }
        __syncthreads();  // (1) L, M, (I + L_bb)^-1, f of chunk c ready

        // ================= P2 =================
        if constexpr (CONS) {
          cons_p2(c, t0, n);
        } else if constexpr (LOAD) {
          // v of chunk c + 1 into LDS (chunk c's was last read in P1); the
          // loads of q and v of chunk c + 2; PGDN: their share of pass 1
          if (c + 1 < nchunks) stash_v();
          if constexpr (!REG && OUT) fetch_q(c + 2);
          fetch_v(c + 2);
          if constexpr (PG) {
            if (c + 1 < nchunks) gains1(c + 1);
          } else {
            if (c + 1 < nchunks) tiles_off(c + 1);  // raw products, scaled in P1 of c + 1
          }
        } else {
          if (c + 1 < nchunks) {
            if constexpr (REG) {
              tiles(c + 1);  // raw products, scaled in P3 (diagonal) and P1 of c + 1
              tiles_off(c + 1);
              diag_gains(c + 1, n1);
            } else {
              gains1(c + 1);  // PGDN statistic pass 1 (and the decay) of chunk c + 1
            }
          }
        }
        __syncthreads();  // (2) REG: raw tiles of chunk c + 1; PGDN: its pass 1

        // ================= P3 =================
        if constexpr (CONS) {
          cons_p3(c);
          // the state entering chunk c + 1: the stores have the next two
          // phases to drain before the next update rewrites S
          if (!OUT && a.S_ck && c + 1 < nchunks) store_ck(c + 1);
        } else if constexpr (LOAD) {
          // REG: the gates and q of chunk c + 2 into LDS (their parity's last
          // readers - regains and diag_gains of chunk c, its Q S - are done);
          // PGDN: their share of pass 2
          if constexpr (REG) {
            stash_gates(c + 2, ntok(c + 2));
            if (OUT && c + 2 < nchunks) stash_q(c + 2);
          } else if (c + 1 < nchunks) {
            gains2(c + 1);
          }
        } else {
          if (c + 1 < nchunks) {
            if constexpr (REG) scale_diag(c + 1);
            else gains2(c + 1);  // PGDN pass 2: the write vectors of chunk c + 1
          }
        }
        __syncthreads();  // (3) chunk c + 1: tiles (REG) or gains (PGDN) ready; S updated
      }

    }

    // ---------------- final state and statistic (neither for a head whose
    // decay left the range of the chunk form: the tokenwise pass that follows
    // writes them, from S0 and aux0 as they are)
    const bool oor = CD && sm.oor;
    if constexpr (CONS) {
      float* fin = xfer ? a.S_final_x : a.S_final;
      if (fin && !oor) {
        float* base = fin + s_lane;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) base[(KL::sigma_channel(dt, 0, i)) * sstride] = S[dt][i];
      }
    } else if constexpr (PROD) {
      if ((PG || KD) && !oor && a.aux_final && slice == 0 && ptid < DK)
        a.aux_final[static_cast<long>(bh) * DK + ptid] = sm.acarry[ptid];
      if (ISO && !oor && a.aux_final && slice == 0 && ptid == 0) a.aux_final[bh] = sm.acarry[nchunks & 1];
      if (CD && a.oor && slice == 0 && ptid == 0) a.oor[bh] = oor ? 1 : 0;
    }
  };
  if (wave < 4) {
    run(Role<0>{});
  } else if (wave < 8) {
    run(Role<1>{});
  } else {
    run(Role<2>{});
  }
}

// Two entry points over the same body.  The one for the scalar-decay gains
// with an output (KLA, GDN, explicit w, PGDN) states that three wavefronts
// per SIMD is its occupancy (768 threads per workgroup allow no more): the
// compiler's scheduler then keeps the LDS reads of the consumers' products
// ahead of their MFMAs instead of waiting on each in turn (measured: the
// consumers' K S, Q S phase from 1.99 K to 1.56 K cycles per chunk, the KLA
// chunk step 3% shorter, PGDN 2.6%).  The other instances keep the default:
// the KDN modes compile to the same registers either way, and the
// no-output instances would spill.
template <int DK, int GAIN, bool OUT>
__global__ __launch_bounds__(WS_THREADS) __attribute__((amdgpu_waves_per_eu(3, 3))) void
chunk_fwd_ws_kernel(ChunkArgs a) {
  chunk_fwd_ws_body<DK, GAIN, OUT>(a);
}
template <int DK, int GAIN, bool OUT>
__global__ __launch_bounds__(WS_THREADS) void chunk_fwd_ws_scan_kernel(ChunkArgs a) {
  chunk_fwd_ws_body<DK, GAIN, OUT>(a);
}

}  // namespace ws

template <int DK, int GAIN, bool OUT>
static hipError_t launch_ws_inst(const ChunkArgs& a, hipStream_t st) {
  using Sm = ws::Smem<DK, GAIN>;
  static_assert(sizeof(Sm) <= 160 * 1024, "LDS budget");
  constexpr bool REG = GAIN == GAIN_KLA || GAIN == GAIN_GDN || GAIN == GAIN_EXPLICIT;
  auto kern = [] {
    if constexpr ((REG || GAIN == GAIN_PGDN) && OUT) return ws::chunk_fwd_ws_kernel<DK, GAIN, OUT>;
    else return ws::chunk_fwd_ws_scan_kernel<DK, GAIN, OUT>;
  }();
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       static_cast<int>(sizeof(Sm)));
  if (err != hipSuccess) return err;
  dim3 grid(static_cast<unsigned>(((a.dv + a.xcols) / ws::BV) * a.B * a.H));
  hipLaunchKernelGGL(kern, grid, dim3(ws::WS_THREADS), sizeof(Sm), st, a);
  return hipGetLastError();
}

// launches without an output (a.o == NULL) take the instance that leaves out
// Q S and M U
template <int DK, int GAIN>
static hipError_t launch_ws_one(const ChunkArgs& a, hipStream_t st) {
  return a.o ? launch_ws_inst<DK, GAIN, true>(a, st) : launch_ws_inst<DK, GAIN, false>(a, st);
}

// bf16 io, scalar decay, gains KLA / GDN / PGDN / explicit.
hipError_t launch_chunk_fwd_bf16_scalar(const ChunkArgs& a, int gain, hipStream_t st) {
#define DN_WS(DK)                                                        \
  switch (gain) {                                                        \
    case GAIN_KLA: return launch_ws_one<DK, GAIN_KLA>(a, st);             \
    case GAIN_GDN: return launch_ws_one<DK, GAIN_GDN>(a, st);             \
    case GAIN_PGDN: return launch_ws_one<DK, GAIN_PGDN>(a, st);           \
    case GAIN_EXPLICIT: return launch_ws_one<DK, GAIN_EXPLICIT>(a, st);   \
    default: return hipErrorInvalidValue;                                \
  }
  if (a.dk == 128) {
    DN_WS(128)
  }
  DN_WS(64)
#undef DN_WS
}

// bf16 io, per-channel decay: diagonal or isotropic KDN, KLA, GDN (KDA),
// explicit w.  (PGDN with per-channel decay, PKDA, takes the generic kernel.)
template <int DK>
static hipError_t launch_ws_channel(const ChunkArgs& a, int gain, hipStream_t st) {
  switch (gain) {
    case GAIN_KDN: return launch_ws_one<DK, GAIN_KDN>(a, st);
    case GAIN_KDN_ISO: return launch_ws_one<DK, GAIN_KDN_ISO>(a, st);
    case GAIN_KLA: return launch_ws_one<DK, GAIN_KLA_CD>(a, st);
    case GAIN_GDN: return launch_ws_one<DK, GAIN_GDN_CD>(a, st);
    case GAIN_EXPLICIT: return launch_ws_one<DK, GAIN_EXPLICIT_CD>(a, st);
    default: return hipErrorInvalidValue;
  }
}
hipError_t launch_chunk_fwd_bf16_channel(const ChunkArgs& a, int gain, hipStream_t st) {
  return a.dk == 128 ? launch_ws_channel<128>(a, gain, st) : launch_ws_channel<64>(a, gain, st);
}

}  // namespace dn
