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
  const void *q, *k, *v;
  GateArgs g;
  const float* S0;    // nullable
  const float* aux0;  // nullable
  void* o;
  float* S_final;    // nullable
  float* aux_final;  // nullable
};

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
// bf16 io, scalar decay, gains KLA / GDN / PGDN / explicit (chunk_fwd_bf16.hip)
hipError_t launch_chunk_fwd_bf16_scalar(const ChunkArgs& a, int gain, hipStream_t st);
// bf16 io, diagonal or isotropic KDN with per-channel decay (chunk_fwd_ws.hip)
hipError_t launch_chunk_fwd_bf16_kdn(const ChunkArgs& a, int gain, hipStream_t st);
hipError_t launch_gain_prep(const GainPrepArgs& a, int io_bf16, int gain, bool channel,
                            hipStream_t st);

}  // namespace dn
