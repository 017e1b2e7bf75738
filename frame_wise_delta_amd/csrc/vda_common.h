// Internal definitions shared by the libvda HIP kernels and host code.
// gfx950 (CDNA4) only: 64-lane wavefronts, MFMA f32_16x16x32 on 16-bit
// operands with float32 accumulation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vda.h"

namespace vda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kThreads = 256;  // every kernel runs 4 wavefronts of 64 lanes

// ----------------------------------------------------------------- MFMA --
// D(16x16) += A(16x32) * B(32x16).  Lane l holds A row (l % 16), B column
// (l % 16), with the eight k values 8*(l/16) .. 8*(l/16)+7; the result lane l
// holds D rows 4*(l/16) .. 4*(l/16)+3 of column (l % 16).
__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------- conversions --
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// float -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ __bf16 bits_to_bf16(uint32_t b) {
  return __builtin_bit_cast(__bf16, (uint16_t)b);
}
// x = hi + lo with hi, lo bfloat16: |x - hi - lo| <= 2^-17 |x| (about).
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  uint32_t h = f32_to_bf16_bits(x);
  float hf = bf16_bits_to_f32(h);
  hi = bits_to_bf16(h);
  lo = bits_to_bf16(f32_to_bf16_bits(x - hf));
}

// Element type tags for the input / output tensors.
struct InF32 { typedef float T; static constexpr int bytes = 4; };
struct InBF16 { typedef u16 T; static constexpr int bytes = 2; };

// ------------------------------------------------------------ workspace --
// [0, 256): device status word (int32) + padding.
// then, per head h and frame slot f (f < n: scanned frame f; f == n: text),
// N = (I + A)^{-1} (d x d float32) followed by B (d x d float32).
constexpr size_t kWsHeader = 256;

__host__ __device__ inline size_t ws_slot_floats(int d) { return (size_t)2 * d * d; }

}  // namespace vda
