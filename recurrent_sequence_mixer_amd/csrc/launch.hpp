// Internal interface between the host library (dn_api.cpp) and the kernel
// translation units.  Argument blocks are passed to kernels by value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dn {

// Shared gate/parameter block.  Pointer meanings and layouts are those of
// include/dn.h; `log2x` = log2(x) of the PGDN bound.
struct GateArgs {
  const void* alpha;
  const float* eta;
  const float* alphaP;
  const float* betaP;
  const float* mu_log;
  const void* omega;
  const float* r;
  const void* w;
  float eps, log2x, mu_info;
};

struct DecodeArgs {
  int N, H, dk, dv;
  const void *q, *k, *v;
  const void* alpha;
  const float* eta;
  const float* alphaP;
  const float* betaP;
  const float* mu_log;
  const void* omega;
  const float* r;
  const void* w;
  float eps, log2x, mu_info;
  float* S;
  float* aux;
  void* o;
};

struct ChunkArgs {
  int B, H, T, dk, dv;
  const void *q, *k, *v;  // required (transfer slices read no v)
  GateArgs g;
  const float* S0;    // nullable
  const float* aux0;  // nullable
  void* o;            // nullable: no output
  float* S_final;    // nullable
  float* aux_final;  // nullable
  // xcols (0 or dk) more value slices that run from S0 = I with v = 0 and no
  // output, their final state going to S_final_x [B, H, dk, xcols] (the
  // transfer matrices of segments)
  int xcols;
  float* S_final_x;
  // per-channel decay, nullable: oor[b H + h] = 1 for a head whose decay left
  // the range of the chunk form in some chunk (its S_final and aux_final are
  // then not written, its outputs are NaN), else 0
  int* oor = nullptr;
  // the backward's checkpoints, nullable (bf16 io, scalar decay, no output
  // o): the state entering every chunk S_ck [B, H, nch, dk, dv] and the
  // residuals E [B, H, T, dv] of the chunk form, fp32
  float* S_ck = nullptr;
  float* E_ck = nullptr;
};

// Tokenwise forward of the heads flagged by the chunked kernels, and of
// every head for fp32 io at dk = 128 (token_fwd.hip): kernel widths (dk 64 /
// 128, dv a multiple of 64).  A head of [B, H] runs when any of its nflag entries of
// flags [B, H, nflag] is nonzero (flags NULL: every head), from S0 (nullable: zeros) and the
// statistic aux0[(b H + h) aux_seg] (nullable: ones), writing o, S_final and
// aux_final (each nullable).
struct TokenArgs {
  int B, H, T, dk, dv;
  const void *q, *k, *v;
  GateArgs g;
  const float* S0;
  const float* aux0;
  int aux_seg;
  void* o;
  float* S_final;
  float* aux_final;
  const int* flags;
  int nflag;
};
hipError_t launch_token_fwd(const TokenArgs& a, int io_bf16, int gain, bool channel, hipStream_t st);

// Long-sequence forward by segments (segment_combine.hip): per head, the
// entering state of every segment from the segments' transfer matrices A_s
// [B, H nseg, dk, dk] and local end states B_s [B, H nseg, dk, dv].
struct CombineArgs {
  int B, H, nseg, dk, dv;
  const float* A;   // [B, H nseg, dk, dk]
  const float* Bs;  // [B, H nseg, dk, dv]
  const float* S0;  // [B, H, dk, dv], nullable (zeros)
  float* S_in;      // [B, H nseg, dk, dv]
  float* S_final;   // [B, H, dk, dv], nullable
  // nullable: S_final is not written for a head with any of its nseg entries
  // of oor [B, H nseg] set
  const int* oor = nullptr;
};
hipError_t launch_segment_combine(const CombineArgs& a, hipStream_t st);

// Long-sequence forward, PGDN and KDN gains (segment_stats.hip): the gain
// statistic entering every segment.  Per head of [B, H] and channel (one per
// head for isotropic KDN), pieces of lsub tokens (lsub divides T / nseg) are
// summarised into summ [B, H, T / lsub, 3, aph], then applied in order from
// aux0 (nullable: ones) into aux_in [B, H nseg, aph] and aux_final (nullable)
// [B, H, aph].  PGDN also repeats mu_log [H] into mu_seg [H nseg].
struct StatArgs {
  int B, H, T, dk, nseg, lsub, gain;
  int channel;  // per-channel decay (alpha bf16 per channel), else fp32 per token
  const void* k;
  GateArgs g;
  const float* aux0;
  float* summ;
  float* aux_in;
  float* aux_final;
  float* mu_seg;
};
hipError_t launch_segment_stats(const StatArgs& a, hipStream_t st);

struct GainPrepArgs {
  int B, H, T, dk;
  int C;  // chunk length of the per-chunk outputs (g_out, aux_chunk): 32 or 64
  const void* k;
  GateArgs g;
  const float* aux0;  // nullable
  float* w_out;
  uint16_t* w_bf16 = nullptr;  // nullable: w written here in bf16 (RNE) instead of w_out
  float* g_out;      // nullable
  float* aux_chunk;  // nullable
  float* aux_final;  // nullable
};

// Chunked backward (chunk_bwd.hip).  Inputs as ChunkArgs, the write vectors
// w [B, H, T, dk] from the gain scan (bf16 with bf16 io and scalar decay,
// otherwise fp32), and the cotangents dO [B, H, T, dv]
// (io dtype), dS_T [B, H, dk, dv] and daux_T (nullable).  Gradients are fp32:
// dq, dk, dw_acc [B, H, T, dk] and dG ([B, H, T], per channel [B, H, T, dk])
// are accumulated over value slices and must start at zero; dv [B, H, T, dv]
// and dS0 (nullable) are written.  Workspace: the state entering every chunk
// S_ck [B, H, nch, dk, dv] and the residuals E [B, H, T, dv].
enum BwdFuse { FUSE_NONE = 0, FUSE_KLA = 1, FUSE_GDN = 2 };
struct BwdArgs {
  int B, H, T, dk, dv;
  // S_ck and E already hold the forward's checkpoints (written by the
  // forward chunk kernel): the state kernel runs only its reverse sweep
  int ck_given = 0;
  const void *q, *k, *v;
  GateArgs g;
  const void* w;  // [B, H, T, dk]: bf16 with bf16 io and scalar decay, else fp32
  const float* S0;
  const void* dO;
  const float* dS_T;
  float* S_ck;
  float* E;
  float* dq_out;
  float* dk_out;
  float* dv_out;
  float* dw_acc;
  float* dG;
  float* dS0;
  // the split backward (launch_chunk_bwd_split): dS_out of every chunk,
  // transposed [B, H, nch, dv, dk], written by its serial kernel for its tile
  // kernel,
  // and Z = (I + L)^-T W~ of every chunk [B, H, nch, 64, dk] as split bf16
  // pairs (hi in the low half)
  float* dS_ck = nullptr;
  uint32_t* Z_ck = nullptr;
  // the segmented sweep (nseg > 1): segment maps segA [B, H nseg, dk, dk] and
  // segB [B, H nseg, dk, dv], and the chained dS_out of every segment seg_in
  // [B, H nseg, dk, dv], all in segment_combine_kernel's (reversed) order
  int nseg = 1;
  float* segA = nullptr;
  float* segB = nullptr;
  float* seg_in = nullptr;
  // the split path's tile kernel runs the write gain's backward itself
  // (FUSE_KLA or FUSE_GDN; FUSE_NONE: it writes dk and dw_acc for
  // launch_gain_bwd): dk final, deta and dalpha written there, dw_acc and dG
  // not
  int fuse_gain = 0;
  float* deta = nullptr;
  float* dalpha = nullptr;
};
hipError_t launch_chunk_bwd_state(const BwdArgs& a, int io_bf16, bool channel, hipStream_t st);
// bf16 io, scalar decay, S_ck and E written by the forward chunk kernel, dv a
// multiple of 64: the dS-independent solves of every chunk (Z into Z_ck, P
// into dv_out), the serial sweep for dS, then one workgroup per chunk for
// the per-(token, key) gradients, which it writes (no accumulation: dq,
// dk_out, dw_acc and dG need no zeroing)
// part 1: the Z / P kernel and the serial sweep (S_ck and E not read); part 2:
// the tile kernel
hipError_t launch_chunk_bwd_split(const BwdArgs& a, hipStream_t st, int part);

// Back through the gains (chunk_bwd.hip), one workgroup per (b, h): adds the
// gain's part to dk and forms the gates' gradients from dw_acc and dG.
struct GainBwdArgs {
  int B, H, T, dk;
  const void* k;
  GateArgs g;
  const float* aux_chunk;  // the statistic entering every chunk: PGDN A, KDN p
                           // [B, H, nch, dk]; KDN_ISO b [B, H, nch]
  const float* daux_T;     // nullable
  const float* dw_acc;
  const float* dG;
  float* dk_out;           // holds the state part on entry
  float* dalpha;
  float* deta;
  float* dalphaP;
  float* dbetaP;
  float* dmu_log;          // [H], accumulated over batch rows (starts at zero)
  float* dw_out;           // explicit w
  float* domega;           // KDN [B, H, T, dk], KDN_ISO [B, H, T]
  float* dr;               // KDN, KDN_ISO [B, H, T]
  float* daux0;            // nullable
};
hipError_t launch_gain_bwd(const GainBwdArgs& a, int io_bf16, int gain, bool channel,
                           hipStream_t st);
// [outer][rs][cs] -> [outer][rd][cd] (pad.hip): copy where r < rs and
// c < cs, `fill_bits` (the element's bit pattern) elsewhere; esize 2 or 4.
hipError_t launch_reshape3(const void* src, void* dst, long outer, int rs, int cs, int rd, int cd,
                           int esize, uint32_t fill_bits, hipStream_t st);
// Zero n floats (a plain fill kernel, so that callers may capture it).
hipError_t launch_zero(float* p, size_t n, hipStream_t st);

hipError_t launch_decode(const DecodeArgs& a, int io_bf16, int gain, bool channel, hipStream_t st);
hipError_t launch_chunk_fwd(const ChunkArgs& a, int io_bf16, int gain, bool channel,
                            hipStream_t st);
// bf16 io, scalar decay, gains KLA / GDN / PGDN / explicit (chunk_fwd_ws.hip)
hipError_t launch_chunk_fwd_bf16_scalar(const ChunkArgs& a, int gain, hipStream_t st);
// bf16 io, per-channel decay, every gain but PGDN (chunk_fwd_ws.hip)
hipError_t launch_chunk_fwd_bf16_channel(const ChunkArgs& a, int gain, hipStream_t st);
hipError_t launch_gain_prep(const GainPrepArgs& a, int io_bf16, int gain, bool channel,
                            hipStream_t st);

}  // namespace dn
