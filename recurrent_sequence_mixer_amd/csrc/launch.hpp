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
};

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
  const void* k;
  GateArgs g;
  const float* aux0;  // nullable
  float* w_out;
  float* g_out;      // nullable
  float* aux_chunk;  // nullable
  float* aux_final;  // nullable
};

hipError_t launch_decode(const DecodeArgs& a, int io_bf16, int gain, bool channel, hipStream_t st);
hipError_t launch_chunk_fwd(const ChunkArgs& a, int io_bf16, int gain, bool channel,
                            hipStream_t st);
// bf16 io, scalar decay, gains KLA / GDN / PGDN / explicit (chunk_fwd_ws.hip)
hipError_t launch_chunk_fwd_bf16_scalar(const ChunkArgs& a, int gain, hipStream_t st);
// bf16 io, diagonal or isotropic KDN with per-channel decay (chunk_fwd_ws.hip)
hipError_t launch_chunk_fwd_bf16_kdn(const ChunkArgs& a, int gain, hipStream_t st);
hipError_t launch_gain_prep(const GainPrepArgs& a, int io_bf16, int gain, bool channel,
                            hipStream_t st);

}  // namespace dn
