// Frame statistics and factorisation of the VDA frame write.
//
// For every (head, frame) one workgroup computes, over the frame's U tokens,
//   A = K^T Diag(beta) K  and  B = V^T Diag(beta) K
// ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
// Generation", method-steps section, step (3)) on MFMA with float32
// accumulation, then inverts G = I + A in registers with a blocked
// Gauss-Jordan sweep and stores N = G^{-1} and B in the workspace.
//
// Data path: K, V rows are streamed from HBM in 64-token rounds, converted to
// f16 (beta*K is rounded once to f16) and written channel-major into LDS so
// that an MFMA operand lane reads eight consecutive tokens of one channel
// with a single 16-byte LDS load.  The 16-byte token groups of each LDS row
// are XOR-swizzled so that both the transposing writes and the operand reads
// are free of bank conflicts.
//
// Gauss-Jordan: the 16-row strips of G are spread over the four wavefronts
// and stay in MFMA accumulators.  Each of the d/16 block steps inverts the
// 16x16 pivot block E in one wavefront (scalar Gauss-Jordan with lane
// shuffles), forms r' = E^{-1} R and c' = -C E^{-1} on the VALU, and applies
// the rank-16 update G -= C r' on MFMA with bf16 hi/lo splits of both factors
// (four products), which keeps the update accurate to about 2^-16.  G is
// symmetric positive definite (eigenvalues >= 1), so no pivoting is needed;
// a pivot <= 0 or a non-finite value sets a bit of the device status word.
#include "vda_common.h"
#include "vda_kernels.h"

namespace vda {

namespace {

constexpr int kRound = 64;  // tokens per LDS round (two MFMA k-steps of 32)

// Offset (in halves) of the 16-byte group `grp` (8 tokens) of LDS row `row`.
__device__ __forceinline__ int tile_off(int row, int grp) {
  const int swz = (row & 7) ^ ((row >> 3) & 7);
  return row * kRound + ((grp ^ swz) << 3);
}

// Eight tokens x eight consecutive channels of K or V, kept as loaded.
template <class TIN>
struct Stage8;

template <>
struct Stage8<InBF16> {
  uint4 raw[8];
  __device__ __forceinline__ void load(int s, const u16* p, bool valid) {
    raw[s] = valid ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ float get(int s, int c) const {
    const uint32_t w = (c >> 1) == 0 ? raw[s].x : (c >> 1) == 1 ? raw[s].y : (c >> 1) == 2 ? raw[s].z : raw[s].w;
    return bf16_bits_to_f32((c & 1) ? (w >> 16) : (w & 0xffffu));
  }
};

template <>
struct Stage8<InF32> {
  float4 raw[8][2];
  __device__ __forceinline__ void load(int s, const float* p, bool valid) {
    raw[s][0] = valid ? reinterpret_cast<const float4*>(p)[0] : make_float4(0, 0, 0, 0);
    raw[s][1] = valid ? reinterpret_cast<const float4*>(p)[1] : make_float4(0, 0, 0, 0);
  }
  __device__ __forceinline__ float get(int s, int c) const {
    const float4 v = raw[s][c >> 2];
    return (c & 3) == 0 ? v.x : (c & 3) == 1 ? v.y : (c & 3) == 2 ? v.z : v.w;
  }
};

template <int D>
struct PrepSmem {
  // stats phase: channel-major token tiles
  static constexpr int kTile = D * kRound;  // halves
  // factorisation phase (float offsets)
  static constexpr int kR = 0;                  // [16][D]  pivot row strip
  static constexpr int kC = kR + 16 * D;        // [D][16]  pivot column strip
  static constexpr int kE = kC + 16 * D;        // [16][16] pivot block inverse
  static constexpr int kRp = kE + 256;          // [16][D]  r' = E^-1 R
  static constexpr int kCp = kRp + 16 * D;      // [D][16]  c' = -C E^-1
  static constexpr int kRt = kCp + 16 * D;      // [D][16] bf16 hi, then lo, of r'^T
  static constexpr int kFloats = kRt + 16 * D;  // (2 x D x 16 bf16 = D x 16 floats)
  static constexpr int kBytes =
      (3 * kTile * 2 > kFloats * 4) ? 3 * kTile * 2 : kFloats * 4;
};

}  // namespace

template <int D, class TIN>
__global__ __launch_bounds__(kThreads, 2) void prepare_kernel(PrepArgs args) {
  using T = typename TIN::T;
  constexpr int RT = D / 16;              // 16-row tiles
  constexpr int NRW = (RT + 3) / 4;       // row tiles per wavefront
  __shared__ __attribute__((aligned(16))) char smem[PrepSmem<D>::kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;

  const int h = blockIdx.x / args.n_eff;
  const int f = blockIdx.x - h * args.n_eff;
  const bool text = f >= args.n;
  const int U = text ? args.Nt : args.U;
  const T* kp;
  const T* vp;
  const float* bp;
  if (text) {
    kp = static_cast<const T*>(args.kt) + (size_t)h * args.Nt * D;
    vp = static_cast<const T*>(args.vt) + (size_t)h * args.Nt * D;
    bp = args.bt + (size_t)h * args.Nt;
  } else {
    const size_t fr = (size_t)h * args.T + (args.a + f);
    kp = static_cast<const T*>(args.k) + fr * args.U * D;
    vp = static_cast<const T*>(args.v) + fr * args.U * D;
    bp = args.beta + fr * args.U;
  }

  _Float16* sK = reinterpret_cast<_Float16*>(smem);
  _Float16* sBK = sK + PrepSmem<D>::kTile;
  _Float16* sV = sBK + PrepSmem<D>::kTile;

  f32x4 accA[NRW][RT], accB[NRW][RT];
#pragma unroll
  for (int m = 0; m < NRW; ++m)
#pragma unroll
    for (int c = 0; c < RT; ++c) {
      accA[m][c] = f32x4{0, 0, 0, 0};
      accB[m][c] = f32x4{0, 0, 0, 0};
    }

  // ------------------------------------------------------------ stats ----
  constexpr int CG = D / 8;                    // channel groups of 8
  constexpr int TASKS = 2 * (kRound / 8) * CG; // (K|V) x token groups x channel groups
  for (int u0 = 0; u0 < U; u0 += kRound) {
    for (int task = tid; task < TASKS; task += kThreads) {
      const int tensor = task / ((kRound / 8) * CG);
      const int rem = task - tensor * ((kRound / 8) * CG);
      const int tg = rem / CG, cg = rem - (rem / CG) * CG;
      const T* src = tensor == 0 ? kp : vp;
      Stage8<TIN> x;
      float bt[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int u = u0 + tg * 8 + s;
        const bool ok = u < U;
        x.load(s, src + (size_t)u * D + cg * 8, ok);
        bt[s] = (tensor == 0 && ok) ? bp[u] : 0.f;
      }
      _Float16* dst = tensor == 0 ? sK : sV;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        f16x8 pk;
#pragma unroll
        for (int s = 0; s < 8; ++s) pk[s] = (_Float16)x.get(s, c);
        *reinterpret_cast<f16x8*>(dst + tile_off(cg * 8 + c, tg)) = pk;
        if (tensor == 0) {
          f16x8 pb;
#pragma unroll
          for (int s = 0; s < 8; ++s) pb[s] = (_Float16)(bt[s] * x.get(s, c));
          *reinterpret_cast<f16x8*>(sBK + tile_off(cg * 8 + c, tg)) = pb;
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kRound / 32; ++kk) {
      const int grp = kk * 4 + lg;
      f16x8 aK[NRW], aV[NRW];
#pragma unroll
      for (int m = 0; m < NRW; ++m) {
        const int ri = wave + 4 * m;
        if (ri < RT) {
          aK[m] = *reinterpret_cast<const f16x8*>(sK + tile_off(16 * ri + lr, grp));
          aV[m] = *reinterpret_cast<const f16x8*>(sV + tile_off(16 * ri + lr, grp));
        }
      }
#pragma unroll
      for (int cj = 0; cj < RT; ++cj) {
        const f16x8 b = *reinterpret_cast<const f16x8*>(sBK + tile_off(16 * cj + lr, grp));
#pragma unroll
        for (int m = 0; m < NRW; ++m) {
          if (wave + 4 * m < RT) {
            accA[m][cj] = mfma_f16(aK[m], b, accA[m][cj]);
            accB[m][cj] = mfma_f16(aV[m], b, accB[m][cj]);
          }
        }
      }
    }
    __syncthreads();
  }

  // G = I + A; flag non-finite statistics
  int bad = 0;
#pragma unroll
  for (int m = 0; m < NRW; ++m) {
    const int ri = wave + 4 * m;
    if (ri < RT) {
#pragma unroll
      for (int cj = 0; cj < RT; ++cj)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (!__builtin_isfinite(accA[m][cj][e]) || !__builtin_isfinite(accB[m][cj][e])) bad |= VDA_DEV_NONFINITE;
          if (cj == ri && 4 * lg + e == lr) accA[m][cj][e] += 1.0f;
        }
    }
  }

  // B goes to the workspace now; its registers are free during the sweep
  float* out = args.frames + ((size_t)h * args.n_eff + f) * ws_slot_floats(D);
#pragma unroll
  for (int m = 0; m < NRW; ++m) {
    const int ri = wave + 4 * m;
    if (ri < RT) {
#pragma unroll
      for (int cj = 0; cj < RT; ++cj)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          out[D * D + (16 * ri + 4 * lg + e) * D + 16 * cj + lr] = accB[m][cj][e];
    }
  }

  // ------------------------------------------------- Gauss-Jordan sweep ----
  float* sf = reinterpret_cast<float*>(smem);
  float* Rb = sf + PrepSmem<D>::kR;
  float* Cb = sf + PrepSmem<D>::kC;
  float* Eb = sf + PrepSmem<D>::kE;
  float* Rp = sf + PrepSmem<D>::kRp;
  float* Cp = sf + PrepSmem<D>::kCp;
  __bf16* RtH = reinterpret_cast<__bf16*>(sf + PrepSmem<D>::kRt);
  __bf16* RtL = RtH + 16 * D;

  for (int p = 0; p < RT; ++p) {
    // 1. publish the pivot row strip and the pivot column strip
#pragma unroll
    for (int m = 0; m < NRW; ++m) {
      const int ri = wave + 4 * m;
      if (ri < RT) {
        if (ri == p) {
#pragma unroll
          for (int cj = 0; cj < RT; ++cj)
#pragma unroll
            for (int e = 0; e < 4; ++e) Rb[(4 * lg + e) * D + 16 * cj + lr] = accA[m][cj][e];
        }
#pragma unroll
        for (int cj = 0; cj < RT; ++cj)
          if (cj == p) {
#pragma unroll
            for (int e = 0; e < 4; ++e) Cb[(16 * ri + 4 * lg + e) * 16 + lr] = accA[m][cj][e];
          }
      }
    }
    __syncthreads();

    // 2. E^{-1} of the 16x16 pivot block, one wavefront, scalar Gauss-Jordan.
    //    Lane holds E[r][c0 + e], r = lane % 16, c0 = 4 * (lane / 16).
    if (wave == 0) {
      const int r = lane & 15, c0 = 4 * (lane >> 4);
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = Rb[r * D + 16 * p + c0 + e];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float piv = __shfl(x[k & 3], k + 16 * (k >> 2), 64);
        const float colk = __shfl(x[k & 3], r + 16 * (k >> 2), 64);
        float rowk[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) rowk[e] = __shfl(x[e], k + 16 * (lane >> 4), 64);
        if (!(piv > 0.f) || !__builtin_isfinite(piv)) bad |= VDA_DEV_PIVOT;
        const float inv = 1.0f / piv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int c = c0 + e;
          if (r == k)
            x[e] = (c == k) ? inv : x[e] * inv;
          else
            x[e] = (c == k) ? -colk * inv : x[e] - colk * (rowk[e] * inv);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) Eb[r * 16 + c0 + e] = x[e];
    }
    __syncthreads();

    // 3. r' = E^{-1} R (16 x D) and c' = -C E^{-1} (D x 16) on the VALU
    for (int idx = tid; idx < 16 * D; idx += kThreads) {
      const int q = idx / D, j = idx - (idx / D) * D;
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) s = fmaf(Eb[q * 16 + t], Rb[t * D + j], s);
      Rp[q * D + j] = s;
      __bf16 hi, lo;
      split_bf16(s, hi, lo);
      RtH[j * 16 + q] = hi;
      RtL[j * 16 + q] = lo;
    }
    for (int idx = tid; idx < 16 * D; idx += kThreads) {
      const int i = idx >> 4, q = idx & 15;
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) s = fmaf(Cb[i * 16 + t], Eb[t * 16 + q], s);
      Cp[i * 16 + q] = -s;
    }
    __syncthreads();

    // 4. rank-16 update G -= C r' outside the pivot row/column strips
#pragma unroll
    for (int m = 0; m < NRW; ++m) {
      const int ri = wave + 4 * m;
      if (ri < RT && ri != p) {
        bf16x8 a;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 hi, lo;
          split_bf16(-Cb[(16 * ri + lr) * 16 + 8 * (lg & 1) + e], hi, lo);
          a[e] = lg < 2 ? hi : lo;
        }
#pragma unroll
        for (int cj = 0; cj < RT; ++cj) {
          if (cj != p) {
            const bf16x8 bh = *reinterpret_cast<const bf16x8*>(RtH + (16 * cj + lr) * 16 + 8 * (lg & 1));
            const bf16x8 bl = *reinterpret_cast<const bf16x8*>(RtL + (16 * cj + lr) * 16 + 8 * (lg & 1));
            accA[m][cj] = mfma_bf16(a, bh, accA[m][cj]);
            accA[m][cj] = mfma_bf16(a, bl, accA[m][cj]);
          }
        }
      }
    }
    // 5. pivot strips take their Gauss-Jordan values
#pragma unroll
    for (int m = 0; m < NRW; ++m) {
      const int ri = wave + 4 * m;
      if (ri < RT) {
        if (ri == p) {
#pragma unroll
          for (int cj = 0; cj < RT; ++cj)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              accA[m][cj][e] = (cj == p) ? Eb[(4 * lg + e) * 16 + lr] : Rp[(4 * lg + e) * D + 16 * cj + lr];
        } else {
#pragma unroll
          for (int cj = 0; cj < RT; ++cj)
            if (cj == p) {
#pragma unroll
              for (int e = 0; e < 4; ++e) accA[m][cj][e] = Cp[(16 * ri + 4 * lg + e) * 16 + lr];
            }
        }
      }
    }
    __syncthreads();
  }

  // ------------------------------------------------------------ output ----
#pragma unroll
  for (int m = 0; m < NRW; ++m) {
    const int ri = wave + 4 * m;
    if (ri < RT) {
#pragma unroll
      for (int cj = 0; cj < RT; ++cj)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (!__builtin_isfinite(accA[m][cj][e])) bad |= VDA_DEV_NONFINITE;
          out[(16 * ri + 4 * lg + e) * D + 16 * cj + lr] = accA[m][cj][e];
        }
    }
  }
  if (bad) atomicOr(args.status, bad);
}

__global__ void clear_status_kernel(int* status) { *status = 0; }

int launch_prepare(const PrepArgs& a, int d, bool in_f32, hipStream_t stream) {
  if (a.H == 0 || a.n_eff == 0) return 0;
  dim3 grid((unsigned)(a.H * a.n_eff)), block(kThreads);
#define VDA_PREP(DD)                                                                  \
  if (d == DD) {                                                                      \
    if (in_f32)                                                                       \
      hipLaunchKernelGGL((prepare_kernel<DD, InF32>), grid, block, 0, stream, a);     \
    else                                                                              \
      hipLaunchKernelGGL((prepare_kernel<DD, InBF16>), grid, block, 0, stream, a);    \
    return 0;                                                                         \
  }
  VDA_PREP(16) VDA_PREP(32) VDA_PREP(64) VDA_PREP(128)
#undef VDA_PREP
  return -1;
}

void launch_clear_status(int* status, hipStream_t stream) {
  hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(1), 0, stream, status);
}

}  // namespace vda
