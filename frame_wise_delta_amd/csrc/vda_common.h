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
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
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
// D(16x16) += A(16x16) * B(16x16), bf16 operands: lane l holds A row (l % 16)
// and B column (l % 16) with k = 4*(l/16) .. 4*(l/16)+3, i.e. the same layout
// as the result (rows 4*(l/16) .. 4*(l/16)+3 of column l % 16).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4 mfma16_bf16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                    c, 0, 0, 0);
}

// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8), each with its own L2.  xcd_block maps b to a logical index that
// numbers the blocks of XCD 0 first, then those of XCD 1, and so on, so that
// consecutive logical blocks (which share data) run on one XCD.  It is a
// bijection on [0, nb) for any nb.
__device__ __forceinline__ int xcd_block(int b, int nb) {
  const int x = b & 7, j = b >> 3;
  int first = 0;  // logical index of the first block of XCD x
#pragma unroll
  for (int i = 0; i < 7; ++i)
    if (i < x) first += (nb - i + 7) >> 3;
  return first + j;
}

// Workgroup barrier that orders LDS traffic only: outstanding global loads
// and stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---------------------------------------------------------- conversions --
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// float -> bf16, round to nearest even (gfx950 converts in hardware).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ __bf16 bits_to_bf16(uint32_t b) {
  return __builtin_bit_cast(__bf16, (uint16_t)b);
}
// x = hi + lo with hi, lo bfloat16: |x - hi - lo| <= 2^-17 |x| (about).
__device__ __forceinline__ void split_bf16(float x, __bf16& hi, __bf16& lo) {
  hi = (__bf16)x;
  lo = (__bf16)(x - (float)hi);
}

// Fused prep of raw inputs: x / sqrt(||x||^2 + kPrepEps) per token and
// gate = sigmoid(logit).
constexpr float kPrepEps = 1e-6f;
__device__ __forceinline__ float sigmoid_gate(float z) { return __builtin_amdgcn_rcpf(1.f + __expf(-z)); }

// Sum of v over each aligned group of W lanes (W a power of two <= 64), in
// every lane of the group.  W = 16 uses DPP (two quad permutations, then row
// rotations by 4 and 8); other widths use lane shuffles.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (W == 16) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));
  } else {
#pragma unroll
    for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  }
  return v;
}

// ------------------------------------------------------------ index maps --
// Window of query chunk c ("Video DeltaNet: A Video-Native Hybrid Attention
// for Livestream Video Generation", core-method section, paragraph 1: a
// bidirectional window aligned to the 5-frame chunks; the forward scan reads
// the history before it, the reverse scan the history after it): window
// chunks lo..hi = c-w..c+w clipped to [0, C-1]; first and last window frame
// ws, we (we clipped to the last scanned frame); the forward state index
// F = lo (chunks wholly before ws) and the reverse state index R = C-1-hi
// (chunks wholly after we).  a = 1 with anchor frames, n scanned frames,
// P frames per chunk.  The host's index map, the readout and the softmax
// branch all take their windows from this one function.
struct ChunkWindow {
  int lo, hi, ws, we, F, R;
};
__host__ __device__ inline ChunkWindow chunk_window(int c, int C, int w, int P, int a, int n) {
  ChunkWindow r;
  r.lo = c - w > 0 ? c - w : 0;
  r.hi = c + w < C - 1 ? c + w : C - 1;
  r.ws = a + P * r.lo;
  r.we = a + P * (r.hi + 1) - 1;
  if (r.we > a + n - 1) r.we = a + n - 1;
  r.F = r.lo;
  r.R = C - 1 - r.hi;
  return r;
}
// Chunk of frame t (-1 for the anchor frames).
__host__ __device__ inline int frame_chunk_of(int t, int a, int n, int P) {
  const int f = t - a;
  return (f >= 0 && f < n) ? f / P : -1;
}

// Element type tags for the input / output tensors.
struct InF32 { typedef float T; static constexpr int bytes = 4; };
struct InBF16 { typedef u16 T; static constexpr int bytes = 2; };

// ------------------------------------------------------------ workspace --
// [0, 256): device status word (int32) + padding.
// then, per head h and frame slot f (f < n: scanned frame f; f == n: text),
// 8 d^2 bytes: N = (I + A)^{-1} as a d x d f16 array in MFMA fragment order
// (below) in the first 2 d^2 bytes, then (at byte 2 d^2) J = B N as a d x d
// f16 array in the scan's accumulator order (the f16x4 at (R * d/16 + c) *
// 64 + l holds J[16R + 4(l/16) + e][16c + l % 16]).  The comparators use the
// upper half: the Newton path keeps B (f16, row-major) at byte 4 d^2, the
// SANA-WM path B' = B / sqrt(U) there; between their two prepare kernels the
// first half holds the upper-triangle 16x16 tiles of A (float32) in
// accumulator order: tile (ri, cj), cj >= ri, lane l holds
// A[16ri + 4(l/16) + e][16cj + l % 16], e = 0..3, as 16 bytes at float offset
// ((ri * d/16 + cj) * 64 + l) * 4.
constexpr size_t kWsHeader = 256;

__host__ __device__ inline size_t ws_slot_floats(int d) { return (size_t)2 * d * d; }

// Fragment order of N: the 16-byte chunk holding N[j][8c .. 8c+7] (row j,
// k-chunk c) sits at chunk index ((ct * KS + kk) * LG + lg) * 16 + lr with
// ct = j / 16, lr = j % 16, kk = c / 4, lg = c % 4, KS = max(1, d / 32) and
// LG = min(4, d / 8).  A wavefront loading the B operand of one 16-column
// tile and one 32-deep k-step reads 64 consecutive chunks (1 KB).
__host__ __device__ inline int ntile_chunk(int d, int j, int c) {
  const int KS = d >= 32 ? d / 32 : 1;
  const int LG = d >= 32 ? 4 : d / 8;
  return (((j >> 4) * KS + (c >> 2)) * LG + (c & 3)) * 16 + (j & 15);
}

}  // namespace vda
