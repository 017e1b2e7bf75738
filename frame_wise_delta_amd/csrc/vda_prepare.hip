// Frame statistics and factorisation of the VDA frame write, as two kernels.
//
// stats_kernel: for every (head, frame) one workgroup computes, over the
// frame's U tokens,
//   A = K^T Diag(beta) K  and  B = V^T Diag(beta) K
// ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
// Generation", method-steps section, step (3)) on MFMA with float32
// accumulation and stores both in the frame's workspace slot (A in the place
// N will take).  K, V rows are streamed from HBM in 64-token rounds, converted
// to f16 (beta*K is rounded once to f16) and written channel-major into LDS
// so that an MFMA operand lane reads eight consecutive tokens of one channel
// with a single 16-byte LDS load.  The 16-byte token groups of each LDS row
// are XOR-swizzled so that both the transposing writes and the operand reads
// are free of bank conflicts.  The next round's global loads are issued
// before the current round's MFMAs.
//
// gj_kernel: inverts G = I + A in registers with a blocked Gauss-Jordan
// sweep and overwrites A with N = G^{-1} as a bf16 hi/lo pair in the MFMA
// fragment order the scan consumes.  The 16-row strips of G stay in MFMA
// accumulators spread over the four wavefronts.  Block step p (16 pivot
// columns):
//   * the owner of strip p inverts the 16x16 pivot block E with a scalar
//     Gauss-Jordan, one matrix row per lane, the pivot row broadcast by DPP
//     row_newbcast, and forms r' = E^{-1} R on MFMA;
//   * every other strip forms c' = -C E^{-1} on MFMA and applies the rank-16
//     update G -= C r'.
// MFMA products use bf16 hi/lo splits of both factors (four partial
// products), accurate to about 2^-16 relative.  G is symmetric positive
// definite (eigenvalues >= 1), so no pivoting is needed; a pivot <= 0 or a
// non-finite value sets a bit of the device status word.  Splitting the two
// phases lets the latency-bound sweep run at a higher occupancy than the
// bandwidth-bound statistics.
#include <utility>

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

// LDS layout of the factorisation phase (byte offsets).  E^{-1} and r'^T
// are read by every wavefront after the step's barrier, so they are
// double-buffered by step parity; R^T is read by its writer only.  Row
// pitches are padded (24 bf16, 20 floats) so that the 16-byte operand reads
// of 16 consecutive rows are free of LDS bank conflicts.
constexpr int kTP = 24;  // bf16 row pitch of R^T / r'^T ([D][16] data)
constexpr int kFP = 20;  // float row pitch of E^{-1} and the column strips ([16][16] data)
template <int D>
struct GjSmem {
  static constexpr int kRT = 0;                        // [D][kTP] bf16 hi, then lo
  static constexpr int kPar0 = kRT + 2 * D * kTP * 2;  // parity buffers:
  static constexpr int kE = 0;                         //   [16][kFP] f32 E^{-1}
  static constexpr int kRpT = 16 * kFP * 4;            //   [D][kTP] bf16 hi, then lo
  static constexpr int kPar = kRpT + 2 * D * kTP * 2;  //   bytes per parity
  static constexpr int kC = kPar0 + 2 * kPar;          // [4 waves][NRW][16][kFP] f32
  static constexpr int kBytes = kC + 4 * ((D / 16 + 3) / 4) * 16 * kFP * 4;
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Lane K of every 16-lane row, broadcast to the whole row (DPP
// row_newbcast; every lane is written, so the old value is irrelevant).
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x150 + K, 0xF, 0xF, true));
}

// One pivot of the scalar Gauss-Jordan inverse below.  With t = x[K] (this
// row's pivot-column entry) and g = (t - [row is pivot row]) / pivot, every
// column c != K becomes x[c] - g * pivotrow[c]: this is x[c] / pivot on the
// pivot row and the usual elimination elsewhere, one FMA per entry with the
// pivot-row entry as a scalar operand.
template <int K>
__device__ __forceinline__ void gj_pivot(f32x16& x, int r, int& bad) {
  const float piv = row_bcast<K>(x[K]);
  if (!(piv > 0.f) || !__builtin_isfinite(piv)) bad |= VDA_DEV_PIVOT;
  const float inv = __builtin_amdgcn_rcpf(piv);  // v_rcp_f32, 1 ulp
  const float t = x[K];
  const bool prow = (r == K);
  const float ng = -(prow ? t - 1.0f : t) * inv;
  float pr[16];
#pragma unroll
  for (int c = 0; c < 16; ++c)
    if (c != K) pr[c] = row_bcast<K>(x[c]);
#pragma unroll
  for (int c = 0; c < 16; ++c)
    if (c != K) x[c] = fmaf(pr[c], ng, x[c]);
  x[K] = prow ? inv : -t * inv;
}

template <int... Ks>
__device__ __forceinline__ void invert16_impl(f32x16& x, int r, int& bad, std::integer_sequence<int, Ks...>) {
  (gj_pivot<Ks>(x, r, bad), ...);
}

// Scalar Gauss-Jordan inverse of a 16x16 matrix held one row per lane (lane
// l holds row l % 16; the four 16-lane groups hold copies); the result has
// the same layout.
__device__ __forceinline__ void invert16(f32x16& x, int r, int& bad) {
  invert16_impl(x, r, bad, std::make_integer_sequence<int, 16>{});
}

__device__ __forceinline__ float pick4(const f32x16& x, int grp, int e) {
  // x[4 * grp + e] for a lane-dependent grp in 0..3
  return grp == 0 ? x[e] : grp == 1 ? x[4 + e] : grp == 2 ? x[8 + e] : x[12 + e];
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

}  // namespace

// Row pitch (floats) of the 64-row float32 staging buffers: d + 4 puts the
// four 16-lane groups of an accumulator tile (rows 4 apart) on disjoint banks.
template <int D>
constexpr int kSP = D + 4;

// Stage 64 rows of a wavefront-strip-distributed d x d float32 matrix
// (accumulator layout) through LDS and store them row-major, coalesced.
template <int D, int NRW>
__device__ __forceinline__ void store_rows(const f32x4 (&acc)[NRW][D / 16], float* stage, float* dst,
                                           int tid, int wave, int lg, int lr) {
  constexpr int RT = D / 16;
  constexpr int SP = kSP<D>;
#pragma unroll
  for (int m = 0; m < NRW; ++m) {
    const int ri = wave + 4 * m;
    if (ri < RT) {
#pragma unroll
      for (int cj = 0; cj < RT; ++cj)
#pragma unroll
        for (int e = 0; e < 4; ++e) stage[(16 * wave + 4 * lg + e) * SP + 16 * cj + lr] = acc[m][cj][e];
    }
    lds_barrier();
    const int rows = (D - 64 * m) < 64 ? (D - 64 * m) : 64;
    float* d = dst + (size_t)64 * m * D;
    for (int i = tid; i < rows * D / 4; i += kThreads) {
      const int r = i / (D / 4), c4 = i - r * (D / 4);
      reinterpret_cast<float4*>(d)[i] = *reinterpret_cast<const float4*>(stage + r * SP + 4 * c4);
    }
    lds_barrier();
  }
}

template <int D, class TIN>
__global__ __launch_bounds__(kThreads, 2) void stats_kernel(PrepArgs args) {
  using T = typename TIN::T;
  constexpr int RT = D / 16;              // 16-row tiles
  constexpr int NRW = (RT + 3) / 4;       // row tiles per wavefront
  constexpr int kTile = D * kRound;       // halves per LDS token tile
  constexpr int kBytes = (3 * kTile * 2 > 64 * kSP<D> * 4) ? 3 * kTile * 2 : 64 * kSP<D> * 4;
  __shared__ __attribute__((aligned(16))) char smem[kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;

  const int h = blockIdx.x / args.cnt;
  const int f = args.s0 + (blockIdx.x - h * args.cnt);
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
  _Float16* sBK = sK + kTile;
  _Float16* sV = sBK + kTile;

  f32x4 accA[NRW][RT], accB[NRW][RT];
#pragma unroll
  for (int m = 0; m < NRW; ++m)
#pragma unroll
    for (int c = 0; c < RT; ++c) {
      accA[m][c] = f32x4{0, 0, 0, 0};
      accB[m][c] = f32x4{0, 0, 0, 0};
    }

  // One load task per thread and round: 8 tokens x 8 channels of K or V.
  constexpr int CG = D / 8;
  constexpr int TASKS = 2 * (kRound / 8) * CG;  // <= 256
  const bool has_task = tid < TASKS;
  const int tensor = tid / ((kRound / 8) * CG);
  const int trem = tid - tensor * ((kRound / 8) * CG);
  const int tg = trem / CG, cg = trem - (trem / CG) * CG;
  const T* src = tensor == 0 ? kp : vp;
  Stage8<TIN> pre;
  float pbt[8];
  auto fetch = [&](int u0) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int u = u0 + tg * 8 + s;
      const bool ok = has_task && u < U;
      pre.load(s, src + (size_t)u * D + cg * 8, ok);
      pbt[s] = (tensor == 0 && ok) ? bp[u] : 0.f;
    }
  };
  if (U > 0) fetch(0);
  for (int u0 = 0; u0 < U; u0 += kRound) {
    if (has_task) {
      _Float16* dst = tensor == 0 ? sK : sV;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        f16x8 pk;
#pragma unroll
        for (int s = 0; s < 8; ++s) pk[s] = (_Float16)pre.get(s, c);
        *reinterpret_cast<f16x8*>(dst + tile_off(cg * 8 + c, tg)) = pk;
        if (tensor == 0) {
          f16x8 pb;
#pragma unroll
          for (int s = 0; s < 8; ++s) pb[s] = (_Float16)(pbt[s] * pre.get(s, c));
          *reinterpret_cast<f16x8*>(sBK + tile_off(cg * 8 + c, tg)) = pb;
        }
      }
    }
    lds_barrier();
    if (u0 + kRound < U) fetch(u0 + kRound);  // in flight during the MFMAs
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
    lds_barrier();
  }

  int bad = 0;
#pragma unroll
  for (int m = 0; m < NRW; ++m)
#pragma unroll
    for (int cj = 0; cj < RT; ++cj)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (!__builtin_isfinite(accA[m][cj][e]) || !__builtin_isfinite(accB[m][cj][e])) bad |= VDA_DEV_NONFINITE;
  float* slot = args.frames + ((size_t)h * args.n_eff + f) * ws_slot_floats(D);
  float* stage = reinterpret_cast<float*>(smem);
  store_rows<D, NRW>(accA, stage, slot, tid, wave, lg, lr);          // A where N will go
  store_rows<D, NRW>(accB, stage, slot + D * D, tid, wave, lg, lr);  // B
  if (bad) atomicOr(args.status, bad);
}

template <int D>
__global__ __launch_bounds__(kThreads, 4) void gj_kernel(PrepArgs args) {
  constexpr int RT = D / 16;
  constexpr int NRW = (RT + 3) / 4;
  constexpr int kStageA = 64 * kSP<D> * 4;        // float32 A rows
  constexpr int kStageN = 2 * 64 * (D + 8) * 2;    // bf16 N hi and lo rows
  constexpr int kStage = kStageA > kStageN ? kStageA : kStageN;
  constexpr int kBytes = GjSmem<D>::kBytes > kStage ? GjSmem<D>::kBytes : kStage;
  __shared__ __attribute__((aligned(16))) char smem[kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int h = blockIdx.x / args.cnt;
  const int f = args.s0 + (blockIdx.x - h * args.cnt);
  float* slot = args.frames + ((size_t)h * args.n_eff + f) * ws_slot_floats(D);
  int bad = 0;

  // ---- load A (row-major float32) into the accumulator layout, G = I + A
  f32x4 accA[NRW][RT];
  float* stage = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int m = 0; m < NRW; ++m) {
    const int rows = (D - 64 * m) < 64 ? (D - 64 * m) : 64;
    const float* src = slot + (size_t)64 * m * D;
    for (int i = tid; i < rows * D / 4; i += kThreads) {
      const int r = i / (D / 4), c4 = i - r * (D / 4);
      *reinterpret_cast<float4*>(stage + r * kSP<D> + 4 * c4) = reinterpret_cast<const float4*>(src)[i];
    }
    lds_barrier();
    const int ri = wave + 4 * m;
    if (ri < RT) {
#pragma unroll
      for (int cj = 0; cj < RT; ++cj)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = stage[(16 * wave + 4 * lg + e) * kSP<D> + 16 * cj + lr];
          if (cj == ri && 4 * lg + e == lr) v += 1.0f;
          accA[m][cj][e] = v;
        }
    }
    lds_barrier();
  }

  // ---- blocked Gauss-Jordan sweep
  char* gj = smem;
  float* sCw = reinterpret_cast<float*>(gj + GjSmem<D>::kC) + wave * NRW * 16 * kFP;
  // fully unrolled: every accumulator index below is a compile-time constant
#pragma unroll
  for (int p = 0; p < RT; ++p) {
    char* par = gj + GjSmem<D>::kPar0 + (p & 1) * GjSmem<D>::kPar;
    float* sE = reinterpret_cast<float*>(par + GjSmem<D>::kE);  // E^{-1}
    __bf16* sRTh = reinterpret_cast<__bf16*>(gj + GjSmem<D>::kRT);
    __bf16* sRTl = sRTh + D * kTP;
    __bf16* sRpTh = reinterpret_cast<__bf16*>(par + GjSmem<D>::kRpT);
    __bf16* sRpTl = sRpTh + D * kTP;
    const bool owner = (p % 4) == wave;
    const int mp = p / 4;

    // A. owner publishes R^T (hi/lo); every wave stages its column strip
#pragma unroll
    for (int m = 0; m < NRW; ++m) {
      const int ri = wave + 4 * m;
      if (ri >= RT) continue;
      if (ri == p) {
#pragma unroll
        for (int cj = 0; cj < RT; ++cj) {
          bf16x4 hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            __bf16 hh, ll;
            split_bf16(accA[m][cj][e], hh, ll);
            hi[e] = hh;
            lo[e] = ll;
          }
          *reinterpret_cast<bf16x4*>(sRTh + (16 * cj + lr) * kTP + 4 * lg) = hi;
          *reinterpret_cast<bf16x4*>(sRTl + (16 * cj + lr) * kTP + 4 * lg) = lo;
        }
      }
#pragma unroll
      for (int cj = 0; cj < RT; ++cj)
        if (cj == p) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sCw[m * 16 * kFP + (4 * lg + e) * kFP + lr] = accA[m][cj][e];
        }
    }

    // B. owner: E^{-1} (scalar Gauss-Jordan, row lr per lane), r' = E^{-1} R
    if (owner) {
      f32x16 x;
#pragma unroll
      for (int c = 0; c < 16; c += 4) {
        const float4 v = *reinterpret_cast<const float4*>(sCw + mp * 16 * kFP + lr * kFP + c);
        x[c] = v.x; x[c + 1] = v.y; x[c + 2] = v.z; x[c + 3] = v.w;
      }
      invert16(x, lr, bad);
      if (lg == 0) {
#pragma unroll
        for (int c = 0; c < 16; c += 4)
          *reinterpret_cast<float4*>(sE + lr * kFP + c) = make_float4(x[c], x[c + 1], x[c + 2], x[c + 3]);
      }
      bf16x8 aE;  // A operand [Einv_hi | Einv_lo] (row lr)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 hh, ll;
        split_bf16((lg & 1) ? x[8 + e] : x[e], hh, ll);
        aE[e] = lg < 2 ? hh : ll;
      }
      // all operand reads, then all MFMAs, then the stores: the tiles overlap
      bf16x8 rh[RT], rl[RT];
#pragma unroll
      for (int cj = 0; cj < RT; ++cj) {
        rh[cj] = *reinterpret_cast<const bf16x8*>(sRTh + (16 * cj + lr) * kTP + 8 * (lg & 1));
        rl[cj] = *reinterpret_cast<const bf16x8*>(sRTl + (16 * cj + lr) * kTP + 8 * (lg & 1));
      }
      f32x4 rp[RT];
#pragma unroll
      for (int cj = 0; cj < RT; ++cj) {
        rp[cj] = mfma_bf16(aE, rh[cj], f32x4{0, 0, 0, 0});
        rp[cj] = mfma_bf16(aE, rl[cj], rp[cj]);
      }
#pragma unroll
      for (int cj = 0; cj < RT; ++cj) {
        bf16x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          __bf16 hh, ll;
          split_bf16(rp[cj][e], hh, ll);
          hi[e] = hh;
          lo[e] = ll;
        }
        *reinterpret_cast<bf16x4*>(sRpTh + (16 * cj + lr) * kTP + 4 * lg) = hi;
        *reinterpret_cast<bf16x4*>(sRpTl + (16 * cj + lr) * kTP + 4 * lg) = lo;
#pragma unroll
        for (int m = 0; m < NRW; ++m)
          if (m == mp) {
            if (cj == p) {
#pragma unroll
              for (int e = 0; e < 4; ++e) accA[m][cj][e] = pick4(x, lg, e);  // Einv[4lg+e][lr]
            } else {
              accA[m][cj] = rp[cj];
            }
          }
      }
    }
    lds_barrier();

    // C. c' = -C E^{-1} and the rank-16 update G -= C r' outside the pivot strips
    bf16x8 eh, el;  // B operand rows of E^{-1} (E symmetric)
    {
      const float4 v0 = *reinterpret_cast<const float4*>(sE + lr * kFP + 8 * (lg & 1));
      const float4 v1 = *reinterpret_cast<const float4*>(sE + lr * kFP + 8 * (lg & 1) + 4);
      const float ev[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 hh, ll;
        split_bf16(ev[e], hh, ll);
        eh[e] = hh;
        el[e] = ll;
      }
    }
#pragma unroll
    for (int m = 0; m < NRW; ++m) {
      const int ri = wave + 4 * m;
      if (ri < RT && ri != p) {
        bf16x8 aC;  // A operand [-C_hi | -C_lo]
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 hh, ll;
          split_bf16(-sCw[m * 16 * kFP + lr * kFP + 8 * (lg & 1) + e], hh, ll);
          aC[e] = lg < 2 ? hh : ll;
        }
        f32x4 cp = {0, 0, 0, 0};
        cp = mfma_bf16(aC, eh, cp);
        cp = mfma_bf16(aC, el, cp);
#pragma unroll
        for (int cj = 0; cj < RT; ++cj) {
          if (cj == p) {
            accA[m][cj] = cp;
          } else {
            const bf16x8 bh = *reinterpret_cast<const bf16x8*>(sRpTh + (16 * cj + lr) * kTP + 8 * (lg & 1));
            const bf16x8 bl = *reinterpret_cast<const bf16x8*>(sRpTl + (16 * cj + lr) * kTP + 8 * (lg & 1));
            accA[m][cj] = mfma_bf16(aC, bh, accA[m][cj]);
            accA[m][cj] = mfma_bf16(aC, bl, accA[m][cj]);
          }
        }
      }
    }
  }
  lds_barrier();

  // ---- N -> workspace as bf16 hi/lo in fragment order, 64 rows at a time
  //      through LDS (overwrites A)
  // N is symmetric, so each pass stages rows [64m, 64m + 64) of N^T (columns
  // of N): every lane writes four consecutive row entries with one 8-byte store.
  constexpr int NP = D + 8;  // bf16 row pitch of the staging (conflict-free 16-byte reads)
  __bf16* sh = reinterpret_cast<__bf16*>(smem);
  __bf16* sl = sh + 64 * NP;
  __bf16* nhi = reinterpret_cast<__bf16*>(slot);
  __bf16* nlo = nhi + D * D;
#pragma unroll
  for (int m = 0; m < NRW; ++m) {
#pragma unroll
    for (int mm = 0; mm < NRW; ++mm) {
      const int ri = wave + 4 * mm;
      if (ri < RT) {
#pragma unroll
        for (int cj = 4 * m; cj < RT && cj < 4 * m + 4; ++cj) {
          bf16x4 hi, lo;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = accA[mm][cj][e];
            if (!__builtin_isfinite(v)) bad |= VDA_DEV_NONFINITE;
            __bf16 hh, ll;
            split_bf16(v, hh, ll);
            hi[e] = hh;
            lo[e] = ll;
          }
          const int idx = (16 * (cj - 4 * m) + lr) * NP + 16 * ri + 4 * lg;
          *reinterpret_cast<bf16x4*>(sh + idx) = hi;
          *reinterpret_cast<bf16x4*>(sl + idx) = lo;
        }
      }
    }
    lds_barrier();
    // rows [64m, 64m + rows) are whole 16-column tiles, i.e. a contiguous
    // range of fragment-order chunks starting at ntile_chunk(D, 64m, 0)
    const int rows = (D - 64 * m) < 64 ? (D - 64 * m) : 64;
    const int n16 = rows * D / 8;  // 16-byte chunks per array
    const int base = ntile_chunk(D, 64 * m, 0);
    for (int i = tid; i < 2 * n16; i += kThreads) {
      const int which = i >= n16;
      const int q = base + (i - which * n16);  // destination chunk
      constexpr int KS = D >= 32 ? D / 32 : 1;
      constexpr int LG = D >= 32 ? 4 : D / 8;
      const int lrq = q & 15, g = q >> 4;
      const int lgq = g % LG, t2 = g / LG;
      const int kk = t2 % KS, ct = t2 / KS;
      const int j = 16 * ct + lrq, c = 4 * kk + lgq;
      const uint4 v = *reinterpret_cast<const uint4*>((which ? sl : sh) + (j - 64 * m) * NP + 8 * c);
      reinterpret_cast<uint4*>(which ? nlo : nhi)[q] = v;
    }
    lds_barrier();
  }
  if (bad) atomicOr(args.status, bad);
}

__global__ void clear_status_kernel(int* status) { *status = 0; }

int launch_stats(const PrepArgs& a, int d, bool in_f32, hipStream_t stream) {
  if (a.H == 0 || a.cnt == 0) return 0;
  dim3 grid((unsigned)(a.H * a.cnt)), block(kThreads);
#define VDA_STATS(DD)                                                                 \
  if (d == DD) {                                                                      \
    if (in_f32)                                                                       \
      hipLaunchKernelGGL((stats_kernel<DD, InF32>), grid, block, 0, stream, a);       \
    else                                                                              \
      hipLaunchKernelGGL((stats_kernel<DD, InBF16>), grid, block, 0, stream, a);      \
    return 0;                                                                         \
  }
  VDA_STATS(16) VDA_STATS(32) VDA_STATS(64) VDA_STATS(128)
#undef VDA_STATS
  return -1;
}

int launch_gj(const PrepArgs& a, int d, hipStream_t stream) {
  if (a.H == 0 || a.cnt == 0) return 0;
  dim3 grid((unsigned)(a.H * a.cnt)), block(kThreads);
#define VDA_GJ(DD)                                                                    \
  if (d == DD) {                                                                      \
    hipLaunchKernelGGL((gj_kernel<DD>), grid, block, 0, stream, a);                   \
    return 0;                                                                         \
  }
  VDA_GJ(16) VDA_GJ(32) VDA_GJ(64) VDA_GJ(128)
#undef VDA_GJ
  return -1;
}

void launch_clear_status(int* status, hipStream_t stream) {
  hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(1), 0, stream, status);
}

}  // namespace vda
