// Device-side helpers shared by the gfx950 kernels of libdn.so:
// element types, bf16 conversion, vector loads and the MFMA tile wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-byte moves
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 stored as raw bits in memory; conversions are explicit.
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f2bf(float f) {
  bf16 h = static_cast<bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}
// Two floats -> two bf16 (RNE) in one word, a in the low half: a single
// v_cvt_pk_bf16_f32 (a vector conversion; element-wise casts would not fuse).
__device__ __forceinline__ uint32_t pack_bf2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Element-type traits of the operand buffers kept in LDS.
// E = uint16_t: bf16 bits; E = float: fp32.
template <typename E> struct Elem;
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float get(uint16_t x) { return bf2f(x); }
  static __device__ __forceinline__ uint16_t put(float x) { return f2bf(x); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float get(float x) { return x; }
  static __device__ __forceinline__ float put(float x) { return x; }
};

// ---------------------------------------------------------------------------
// 16x16 output tiles on the matrix cores.
//
// Operand storage convention (both A and B): "k-contiguous".  A product
// C[16 x 16] += A[16 x K] * B[K x 16] reads A as rows a[r * lda + k] and B as
// columns b[c * ldb + k], i.e. B is stored transposed.  Every lane loads the
// same k-subset for A and for B, so the contraction is exact whatever slot
// order the instruction uses internally.
//
// Accumulator layout (16x16 f32, 4 values per lane): lane l holds rows
// 4*(l/16) + i, i = 0..3, of column l % 16.
// ---------------------------------------------------------------------------
template <typename E> struct MmaK;  // k-step of one MFMA instruction
template <> struct MmaK<uint16_t> { static constexpr int v = 32; };
template <> struct MmaK<float> { static constexpr int v = 4; };

template <typename E> struct Mma;

template <> struct Mma<uint16_t> {
  using Frag = bf16x8;  // v_mfma_f32_16x16x32_bf16: 8 bf16 per lane
  // Fragment of k-step s from k-contiguous storage: lane l reads row l % 16,
  // k = 32 s + 8 (l / 16) .. +7 (one 16-byte LDS read).
  static __device__ __forceinline__ Frag frag(const uint16_t* p, int ld, int lane, int s) {
    const uint16_t* q = p + (lane & 15) * ld + 32 * s + 8 * (lane >> 4);
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(q));
  }
  static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  // C += A[16 x K] B[K x 16], K a multiple of 32.
  static __device__ __forceinline__ void run(f32x4& c, const uint16_t* a, int lda, const uint16_t* b,
                                             int ldb, int K, int lane) {
#pragma unroll
    for (int s = 0; s < K / 32; ++s) c = mma(frag(a, lda, lane, s), frag(b, ldb, lane, s), c);
  }
};

template <> struct Mma<float> {
  using Frag = float;  // v_mfma_f32_16x16x4_f32: 1 fp32 per lane
  static __device__ __forceinline__ Frag frag(const float* p, int ld, int lane, int s) {
    return p[(lane & 15) * ld + 4 * s + (lane >> 4)];
  }
  static __device__ __forceinline__ f32x4 mma(Frag a, Frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void run(f32x4& c, const float* a, int lda, const float* b,
                                             int ldb, int K, int lane) {
#pragma unroll
    for (int s = 0; s < K / 4; ++s) c = mma(frag(a, lda, lane, s), frag(b, ldb, lane, s), c);
  }
};

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Debug builds (-DDN_DEBUG): every byte of a kernel's LDS is set to all ones
// (NaN as fp32 and as bf16) before the kernel's first LDS access, so that a
// result depending on LDS that no thread wrote turns into NaN in the parity
// tests.  Release builds compile DN_LDS_POISON to nothing.
#ifdef DN_DEBUG
#define DN_LDS_POISON(p, bytes)                                                              \
  do {                                                                                       \
    uint32_t* w_ = reinterpret_cast<uint32_t*>(p);                                           \
    for (unsigned i_ = threadIdx.x; i_ < static_cast<unsigned>((bytes) / 4); i_ += blockDim.x) \
      w_[i_] = 0xFFFFFFFFu;                                                                  \
    __syncthreads();                                                                         \
  } while (0)
#else
#define DN_LDS_POISON(p, bytes) \
  do {                          \
  } while (0)
#endif

// Sum over the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// DPP move within rows of 16 lanes (gfx9 encodings: quad_perm = 2-bit lane
// selectors, row_mirror = 0x140, row_half_mirror = 0x141).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sums of 64 per-lane vectors across the 64 lanes of a wavefront,
// reduce-scattered: on return lane l holds the total of element l.  Each
// halving step pairs a lane with one whose bit D differs and whose higher
// bits agree (xor 32 and 16 by cross-lane shuffles, the row mirrors for 8
// and 4, quad permutes for 2 and 1): the lane keeps half D of its block and
// adds the partner's copy of it.  v is overwritten.
__device__ __forceinline__ float wave_reduce_scatter64(float (&v)[64], int lane) {
  auto step = [&](auto dtag, auto partner) __attribute__((always_inline)) {
    constexpr int D = decltype(dtag)::value;
    const bool hi = (lane & D) != 0;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const float send = hi ? v[i] : v[D + i];
      const float keep = hi ? v[D + i] : v[i];
      v[i] = keep + partner(send);
    }
  };
  step(std::integral_constant<int, 32>{}, [](float x) { return __shfl_xor(x, 32, 64); });
  step(std::integral_constant<int, 16>{}, [](float x) { return __shfl_xor(x, 16, 64); });
  step(std::integral_constant<int, 8>{}, [](float x) { return dpp_move<0x140>(x); });
  step(std::integral_constant<int, 4>{}, [](float x) { return dpp_move<0x141>(x); });
  step(std::integral_constant<int, 2>{}, [](float x) { return dpp_move<0x4E>(x); });
  step(std::integral_constant<int, 1>{}, [](float x) { return dpp_move<0xB1>(x); });
  return v[0];
}
// The same for 32 values: lanes l and l + 32 both end with the wavefront's
// total of element l % 32.
__device__ __forceinline__ float wave_reduce_scatter32(float (&v)[32], int lane) {
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] += __shfl_xor(v[i], 32, 64);
  auto step = [&](auto dtag, auto partner) __attribute__((always_inline)) {
    constexpr int D = decltype(dtag)::value;
    const bool hi = (lane & D) != 0;
#pragma unroll
    for (int i = 0; i < D; ++i) {
      const float send = hi ? v[i] : v[D + i];
      const float keep = hi ? v[D + i] : v[i];
      v[i] = keep + partner(send);
    }
  };
  step(std::integral_constant<int, 16>{}, [](float x) { return __shfl_xor(x, 16, 64); });
  step(std::integral_constant<int, 8>{}, [](float x) { return dpp_move<0x140>(x); });
  step(std::integral_constant<int, 4>{}, [](float x) { return dpp_move<0x141>(x); });
  step(std::integral_constant<int, 2>{}, [](float x) { return dpp_move<0x4E>(x); });
  step(std::integral_constant<int, 1>{}, [](float x) { return dpp_move<0xB1>(x); });
  return v[0];
}

}  // namespace dn
