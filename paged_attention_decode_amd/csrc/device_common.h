// Device-side helpers shared by the libpagedattn kernels (gfx950).
#pragma once

#include "pa_internal.h"

#include <math.h>

// Cache policy of the K/V page loads (gfx940-family buffer instruction bits):
// tiles at or past DecodeArgs::cached_prefix_tokens are loaded non-temporal
// (streamed through the caches); earlier tiles, where prefix-cached blocks
// shared between sequences live, use the default policy so sequences sharing
// them can hit in the last-level cache.
constexpr int kPolicyDefault = 0;
constexpr int kPolicyStream = 2;  // nt
// Third descriptor word of a raw 32-bit buffer resource on gfx9-family GPUs.
constexpr int kRsrcWord3 = 0x00020000;
// Tiles whose K/V loads are in flight ahead of the tile being computed (1 or 2).
#ifndef PA_PREFETCH_TILES
#define PA_PREFETCH_TILES 1
#endif

namespace pa {
namespace dev {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef unsigned int u4 __attribute__((ext_vector_type(4)));
typedef short s4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef _Float16 h4 __attribute__((__vector_size__(4 * sizeof(_Float16))));
typedef _Float16 h8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef __bf16 b8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef unsigned int u2 __attribute__((__vector_size__(2 * sizeof(unsigned int))));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef _Float16 hf2 __attribute__((ext_vector_type(2)));

template <int DT, int D>
struct Cfg {
  static constexpr int kE = (DT == kF32) ? 4 : 2;  // bytes per element
  static constexpr int kX = 16 / kE;               // elements per 16-byte chunk
  static constexpr int kChunks = D / kX;           // 16-byte chunks per key row
  static constexpr int kLoads = kChunks / 4;       // 16-byte loads per lane per tile (K, and V)
  static constexpr int kAcc = D / 16;              // 16x16 accumulator tiles of O^T
  // Deeper prefetch only where the extra register set still fits two wavefronts per SIMD.
  static constexpr int kPrefetch = (PA_PREFETCH_TILES >= 2 && kLoads <= 4) ? 2 : 1;
};

__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  // Round to nearest even; inputs here are finite.
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// fp16 inputs: the softmax weights are computed times 2^(15 - max_weight_log2) (the same factor
// in the running sum, so nothing else changes), which keeps them in fp16's normal range when they
// are rounded to fp16 for the second product (decode: value + remainder; prefill: one rounding).
// Unscaled, a weight below 2^-14 of the running maximum would be an fp16 subnormal, with absolute
// precision 2^-25 only, and many such weights could add up to a visible error. Decode weights are
// at most 1 before scaling (2^15 after); prefill allows 2^8 (lazy rescale) and scales by 2^7.
template <int DT>
constexpr float weight_log2_scale(int max_weight_log2) {
  return DT == kF16 ? (float)(15 - max_weight_log2) : 0.0f;
}

// Maximum over lanes l, l^16, l^32 and l^48 (the four 16-lane rows), with gfx950's row-swap
// instructions: each swap leaves lane l's value and its partner's in the two results.
// The maxima are IEEE-2019 `maximum` (gfx950 has it natively, with a three-input form): unlike
// fmaxf it needs no NaN-quieting instruction on inputs the compiler cannot prove canonical, such
// as matrix-core results.
__device__ __forceinline__ float max_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float fmax8(const float (&x)[8]) {
  const float a = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0], x[1]), x[2]);
  const float b = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[3], x[4]), x[5]);
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), __builtin_elementwise_maximum(x[6], x[7]));
}

// Read-only view of a table that no kernel writes while it runs (block tables): uniform reads
// through it become scalar loads, which wait on their own counter instead of the vector one.
typedef const __attribute__((address_space(4))) int32_t const_i32;

// 16-byte load at byte `off` of a buffer resource, with cache policy POL.
template <int POL>
__device__ __forceinline__ u4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, POL));
}

// 8-byte load at byte `off` of a buffer resource, with cache policy POL.
template <int POL>
__device__ __forceinline__ u2 buf_load8(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(u2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, POL));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, kRsrcWord3);
}

__device__ __forceinline__ int clamp_len(int L, int max_len) {
  return L < 0 ? 0 : (L > max_len ? max_len : L);
}

// Write 8 consecutive output values (d0 .. d0+7) of one head row.
template <int DT>
__device__ __forceinline__ void store8(void* out, int64_t idx, const float (&v)[8], bool out_f32) {
  if (out_f32) {
    f4* p = reinterpret_cast<f4*>(reinterpret_cast<float*>(out) + idx);
    p[0] = f4{v[0], v[1], v[2], v[3]};
    p[1] = f4{v[4], v[5], v[6], v[7]};
  } else if constexpr (DT == kBF16) {
    u4 w;
    w.x = bf16_bits_rne(v[0]) | (bf16_bits_rne(v[1]) << 16);
    w.y = bf16_bits_rne(v[2]) | (bf16_bits_rne(v[3]) << 16);
    w.z = bf16_bits_rne(v[4]) | (bf16_bits_rne(v[5]) << 16);
    w.w = bf16_bits_rne(v[6]) | (bf16_bits_rne(v[7]) << 16);
    *reinterpret_cast<u4*>(reinterpret_cast<uint16_t*>(out) + idx) = w;
  } else if constexpr (DT == kF16) {
    h8 w;
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = (_Float16)v[j];
    *reinterpret_cast<h8*>(reinterpret_cast<_Float16*>(out) + idx) = w;
  }
}

// Write 4 consecutive output values (d0 .. d0+3) of one head row.
template <int DT>
__device__ __forceinline__ void store4(void* out, int64_t idx, const float (&v)[4], bool out_f32) {
  if (out_f32) {
    *reinterpret_cast<f4*>(reinterpret_cast<float*>(out) + idx) = f4{v[0], v[1], v[2], v[3]};
  } else if constexpr (DT == kBF16) {
    u2 w;
    w[0] = bf16_bits_rne(v[0]) | (bf16_bits_rne(v[1]) << 16);
    w[1] = bf16_bits_rne(v[2]) | (bf16_bits_rne(v[3]) << 16);
    *reinterpret_cast<u2*>(reinterpret_cast<uint16_t*>(out) + idx) = w;
  } else if constexpr (DT == kF16) {
    h4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j) w[j] = (_Float16)v[j];
    *reinterpret_cast<h4*>(reinterpret_cast<_Float16*>(out) + idx) = w;
  }
}

}  // namespace dev
}  // namespace pa
