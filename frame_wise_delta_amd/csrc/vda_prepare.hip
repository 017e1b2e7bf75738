// Frame statistics and factorisation of the VDA frame write.
//
// frame_kernel (the path): for every (head, frame slot) one workgroup
// computes A = K^T Diag(beta) K and B = V^T Diag(beta) K over the frame's U
// tokens ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream
// Video Generation", method-steps section, step (3)), factorises I + A by a
// blocked Gauss-Jordan sweep with B^T as right-hand side, and stores
// N = (I + A)^{-1} and J = B N in the frame's workspace slot; A and B never
// leave the workgroup.  K and V rows are streamed from HBM in 64-token
// rounds, converted to f16 and written channel-major into LDS so that an
// MFMA operand lane reads eight consecutive tokens of one channel with a
// single 16-byte LDS load.  The 16-byte token groups of each LDS row are
// XOR-swizzled so that both the transposing writes and the operand reads are
// free of bank conflicts.  The next round's global loads are issued before
// the current round's MFMAs.
//
// stats_kernel (the comparators): the same statistics, stored as the
// upper-triangle tiles of A (float32) and B (f16, row-major) for the
// SANA-WM transition (sana_kernel) and the Newton-iteration inverse
// (ns_kernel), which read them back.
#include <utility>

#include "vda_common.h"
#include "vda_kernels.h"

namespace vda {

namespace {

constexpr int kRound = 64;  // tokens per LDS round (two MFMA k-steps of 32)

// Offset (in halves) of the 16-byte group `grp` (8 tokens) of LDS row `row`.
// The swizzle spreads both access patterns over distinct banks: the
// transposing writes (eight lanes per pass, rows 8 apart, one group) and the
// operand reads (32 lanes per pass, 16 consecutive rows, two groups).
__device__ __forceinline__ int tile_off(int row, int grp) {
  const int swz = ((row >> 1) ^ (row >> 3)) & 7;
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
  // sum of squares of token s's eight values, straight from the packed words
  __device__ __forceinline__ float sumsq(int s) const {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    float a = 0.f;
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, raw[s].x), __builtin_bit_cast(b2, raw[s].x), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, raw[s].y), __builtin_bit_cast(b2, raw[s].y), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, raw[s].z), __builtin_bit_cast(b2, raw[s].z), a, false);
    a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, raw[s].w), __builtin_bit_cast(b2, raw[s].w), a, false);
    return a;
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
  __device__ __forceinline__ float sumsq(int s) const {
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) a = fmaf(get(s, c), get(s, c), a);
    return a;
  }
};

// ---- helpers of the factorisation --------------------------------------

// Lane K of every 16-lane row, broadcast to the whole row (DPP
// row_newbcast; every lane is written, so the old value is irrelevant).
template <int K>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x150 + K, 0xF, 0xF, true));
}

// Row R (lanes 16R .. 16R+15) of v, broadcast to all four 16-lane rows: lane
// l gets v of lane 16R + l % 16.  permlane16_swap(v, v) yields the rows
// (0,0,2,2) and (1,1,3,3); permlane32_swap(u, u) yields (0,1,0,1) and (2,3,2,3).
template <int R>
__device__ __forceinline__ float group_bcast(float v) {
  const unsigned b = __float_as_uint(v);
  const auto s16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  const unsigned u = (R & 1) ? s16[1] : s16[0];
  const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float((R & 2) ? s32[1] : s32[0]);
}

// One pivot of the in-place Gauss-Jordan inverse of a 16x16 matrix W held
// four columns per lane: lane (n, g) = (l % 16, l / 16) holds W[n][4g .. 4g+3].
// With t = W[n][K] and g' = (t - [n == K]) / W[K][K], every column c != K
// becomes W[n][c] - g' W[K][c] (this is W[K][c] / W[K][K] on the pivot row
// and the usual elimination elsewhere), and column K becomes 1 / W[K][K] on
// the pivot row and -t / W[K][K] elsewhere.
template <int K>
__device__ __forceinline__ void gj_pivot(f32x4& y, int n, int g, int& bad) {
  constexpr int KG = K >> 2, KE = K & 3;
  const float t = group_bcast<KG>(y[KE]);  // W[n][K]
  const float piv = row_bcast<K>(t);       // W[K][K]
  if (!(piv > 0.f) || !__builtin_isfinite(piv)) bad |= VDA_DEV_PIVOT;
  const float inv = __builtin_amdgcn_rcpf(piv);  // v_rcp_f32, 1 ulp
  const bool prow = n == K;
  const float ng = -(prow ? t - 1.0f : t) * inv;
  float pr[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) pr[e] = row_bcast<K>(y[e]);  // W[K][4g + e]
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = fmaf(pr[e], ng, y[e]);
  const float colk = prow ? inv : -t * inv;
  y[KE] = g == KG ? colk : y[KE];
}

template <int... Ks>
__device__ __forceinline__ void invert16_impl(f32x4& y, int n, int g, int& bad, std::integer_sequence<int, Ks...>) {
  (gj_pivot<Ks>(y, n, g, bad), ...);
}

// In-place inverse of the 16x16 matrix W held four columns per lane (above).
__device__ __forceinline__ void invert16(f32x4& y, int n, int g, int& bad) {
  invert16_impl(y, n, g, bad, std::make_integer_sequence<int, 16>{});
}

}  // namespace

// Row tile m of wavefront `wave` in the statistics kernel.  With eight row
// tiles (d = 128) the wavefronts take the pairs {w, 7 - w}, so each one owns
// exactly nine of the 36 upper-triangle tiles of the symmetric A (tile (i, j),
// j >= i, is computed by the wavefront owning row tile i); otherwise row
// tiles wave, wave + 4, ...
template <int RT>
__device__ __forceinline__ int row_tile(int wave, int m) {
  if constexpr (RT == 8) return m == 0 ? wave : RT - 1 - wave;
  return wave + 4 * m;
}

// Row pitch (floats) of the 64-row float32 staging buffers: d + 4 puts the
// four 16-lane groups of an accumulator tile (rows 4 apart) on disjoint banks.
template <int D>
constexpr int kSP = D + 4;

// Stage 64 rows of a wavefront-strip-distributed d x d float32 matrix
// (accumulator layout) through LDS and store them row-major as f16,
// coalesced.
template <int D, int NRW>
__device__ __forceinline__ void store_rows(const f32x4 (&acc)[NRW][D / 16], float* stage, _Float16* dst,
                                           int tid, int wave, int lg, int lr) {
  constexpr int RT = D / 16;
  constexpr int SP = kSP<D>;
#pragma unroll
  for (int m = 0; m < NRW; ++m) {
    const int ri = row_tile<RT>(wave, m);  // within rows 64 m .. 64 m + 63
    if (ri < RT) {
#pragma unroll
      for (int cj = 0; cj < RT; ++cj)
#pragma unroll
        for (int e = 0; e < 4; ++e) stage[(16 * (ri - 4 * m) + 4 * lg + e) * SP + 16 * cj + lr] = acc[m][cj][e];
    }
    lds_barrier();
    const int rows = (D - 64 * m) < 64 ? (D - 64 * m) : 64;
    _Float16* d = dst + (size_t)64 * m * D;
    for (int i = tid; i < rows * D / 4; i += kThreads) {
      const int r = i / (D / 4), c4 = i - r * (D / 4);
      const float4 v = *reinterpret_cast<const float4*>(stage + r * SP + 4 * c4);
      reinterpret_cast<f16x4*>(d)[i] = f16x4{(_Float16)v.x, (_Float16)v.y, (_Float16)v.z, (_Float16)v.w};
    }
    lds_barrier();
  }
}

template <int D, class TIN, bool PREP>
__global__ __launch_bounds__(kThreads, 2) void stats_kernel(PrepArgs args) {
  using T = typename TIN::T;
  constexpr int RT = D / 16;              // 16-row tiles
  constexpr int NRW = (RT + 3) / 4;       // row tiles per wavefront
  constexpr int kTile = D * kRound;       // halves per LDS token tile
  constexpr int kBytes = (3 * kTile * 2 > 64 * kSP<D> * 4) ? 3 * kTile * 2 : 64 * kSP<D> * 4;
  __shared__ __attribute__((aligned(16))) char smem[kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    if (PREP && tensor == 0) {
      // raw keys: 1 / ||k|| per token over the CG threads of its row, and
      // beta = sigmoid(logit); the K operand becomes k / ||k||, beta*K beta k / ||k||
      float rn[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        rn[s] = __builtin_amdgcn_rsqf(group_sum<CG>(pre.sumsq(s)) + kPrepEps);
        pbt[s] = sigmoid_gate(pbt[s]) * rn[s];
      }
      if (has_task) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          f16x8 pk, pb;
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const float x = pre.get(s, c);
            pk[s] = (_Float16)(x * rn[s]);
            pb[s] = (_Float16)(pbt[s] * x);
          }
          *reinterpret_cast<f16x8*>(sK + tile_off(cg * 8 + c, tg)) = pk;
          *reinterpret_cast<f16x8*>(sBK + tile_off(cg * 8 + c, tg)) = pb;
        }
      }
    } else if (has_task) {
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
        const int ri = row_tile<RT>(wave, m);
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
          const int ri = row_tile<RT>(wave, m);
          if (ri < RT) {
            if (cj >= ri) accA[m][cj] = mfma_f16(aK[m], b, accA[m][cj]);  // upper triangle only
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
  // A where N will go: the upper-triangle tiles, straight from the accumulators
#pragma unroll
  for (int m = 0; m < NRW; ++m) {
    const int ri = row_tile<RT>(wave, m);
    if (ri < RT) {
#pragma unroll
      for (int cj = 0; cj < RT; ++cj)
        if (cj >= ri) *reinterpret_cast<f32x4*>(slot + ((size_t)(ri * RT + cj) * 64 + lane) * 4) = accA[m][cj];
    }
  }
  float* stage = reinterpret_cast<float*>(smem);
  store_rows<D, NRW>(accB, stage, reinterpret_cast<_Float16*>(slot + D * D), tid, wave, lg, lr);  // B (f16)
  if (bad) atomicOr(args.status, bad);
}

// Own column tiles of wavefront w in the frame kernel: w and w + 4 (those
// below RT).  Column p of every step of the sweep belongs to wavefront p % 4.
template <int RT>
constexpr int kOwnCols = (RT + 3) / 4;

// f16 hi/lo pair of four floats: hi = v rounded to f16, lo = v - hi (exact)
// rounded to f16, so hi + lo holds v to about 2^-22 relative (down to the
// f16 subnormal spacing 2^-24 in absolute terms).
__device__ __forceinline__ void split_f16(f32x4 v, f16x4& hi, f16x4& lo) {
  hi = __builtin_convertvector(v, f16x4);
  lo = __builtin_convertvector(v - __builtin_convertvector(hi, f32x4), f16x4);
}
__device__ __forceinline__ f16x8 cat_f16(f16x4 a, f16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f16x8 neg_f16(f16x8 a) {
  uint4 u = __builtin_bit_cast(uint4, a);
  u.x ^= 0x80008000u;
  u.y ^= 0x80008000u;
  u.z ^= 0x80008000u;
  u.w ^= 0x80008000u;
  return __builtin_bit_cast(f16x8, u);
}

// Products of 16 x 16 float32 tiles on the K = 32 f16 MFMA, accurate to
// about 2^-22: a left factor L enters as the A operand [L_hi | L_lo] (lane
// (m, g) holds L[m][4g .. 4g+3] in both halves), a right factor R as the two
// B operands [R_hi | R_hi] and [R_lo | R_lo] (lane (n, g) holds
// R[4g .. 4g+3][n]), so the two MFMAs sum (L_hi + L_lo)(R_hi + R_lo) over the
// 16-deep k.  An accumulator tile Z (lane (n, g) holds Z[4g + e][n]) is its
// own right operand; a tile read from LDS can be laid out as either.
struct RightF16 {
  f16x8 hh, ll;
};
__device__ __forceinline__ f16x8 left_f16(f32x4 v) {
  f16x4 h, l;
  split_f16(v, h, l);
  return cat_f16(h, l);
}
__device__ __forceinline__ RightF16 right_f16(f32x4 v) {
  f16x4 h, l;
  split_f16(v, h, l);
  return RightF16{cat_f16(h, h), cat_f16(l, l)};
}
__device__ __forceinline__ f32x4 mul_f16(f16x8 left, const RightF16& r, f32x4 acc) {
  acc = mfma_f16(left, r.hh, acc);
  return mfma_f16(left, r.ll, acc);
}
// Right operands [I | 0], [0 | I] and [-I | -I] in lane (n, g): k = 4g + e.
__device__ __forceinline__ f16x8 eye_f16(int n, int g, int half, float val) {
  f16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (_Float16)(((e >> 2) == half || half < 0) && 4 * g + (e & 3) == n ? val : 0.f);
  return r;
}
// The left operand [Z_hi | Z_lo] of a tile Z held in accumulator layout:
// the accumulator registers, read as an A operand, are Z^T, so a product
// with the identity returns Z^T in accumulator layout, i.e. Z in A-operand
// layout; the hi and lo halves are moved separately, exactly.
__device__ __forceinline__ f16x8 to_left_f16(f32x4 z, f16x8 eye_hi, f16x8 eye_lo) {
  f16x4 h, l;
  split_f16(z, h, l);
  const f16x8 a = cat_f16(h, l);
  const f32x4 th = mfma_f16(a, eye_hi, f32x4{0, 0, 0, 0});
  const f32x4 tl = mfma_f16(a, eye_lo, f32x4{0, 0, 0, 0});
  return cat_f16(__builtin_convertvector(th, f16x4), __builtin_convertvector(tl, f16x4));
}

// The frame write's statistics and factorisation in one workgroup per (head,
// frame slot) ("Video DeltaNet: A Video-Native Hybrid Attention for
// Livestream Video Generation", method-steps section, step (3): A_t and B_t
// from the frame's tokens, the factorisation of I + A_t, the transition and
// the injection; core-method section, paragraph 2: the frame write
// S_t = (S_{t-1} Diag(alpha_t) + B_t)(I + A_t)^{-1}).  It stores
//   N = (I + A)^{-1}      (f16, the fragment order of the scan's B operand)
//   J = B N               (f16, the scan's accumulator order, at byte 2 d^2)
// so that the scan computes S_t = (S_{t-1} Diag(alpha_t)) N_t + J_t.  J
// rather than B is stored because every quantity the scan then reads is of
// the size of the state: B itself grows with the conditioning of I + A
// (about by its condition number), and so would the relative effect of any
// rounding of B or of the N that multiplies it.
//
// Statistics.  K and V stream through LDS in 64-token rounds as f16 tiles
// K, beta*K and beta*V (each rounded once to f16; rounding beta*V instead of
// using beta*K for B puts the rounding of B in the span of the keys, where
// N damps it).  Wavefront w owns the column tiles i in {w, w + 4} of
//   T = I + A    (tile (c, i) = sum_u K[u][c] (beta K)[u][i], plus I)
//   X = B        (tile (c, i) = sum_u (beta V)[u][c] K[u][i])
// for every row tile c, in float32 accumulators.
//
// Inverse.  Blocked Gauss-Jordan on G = I + A (symmetric positive definite,
// no pivoting), written for the transpose T = M^T of the working matrix M
// that the wavefronts hold by columns.  Step p, with E^T the tile T[p][p]:
//   Ei^T = (E^T)^{-1}, then for every column i != p
//     T[j][i] -= (T[j][p] Ei^T) T[p][i]   (j != p),
//     T[p][i]  = -Ei^T T[p][i],
//   and column p becomes T[j][p] Ei^T, T[p][p] = Ei^T.
// After the last step T = N^T = N.  The owner of column p inverts the pivot
// tile (scalar Gauss-Jordan, four columns per lane) and stages column p
// through LDS (double-buffered, one barrier per step); every wavefront then
// forms the left factors T[j][p] Ei^T as the transposed products
// Ei (T[j][p])^T, whose accumulator registers are exactly the A operands of
// the left factors, and updates its own columns, the next pivot's column
// first.
//
// Injection.  J = B N as a product: the B tiles of every row tile are
// staged through LDS at once by the owners of their columns (4 d^2 bytes:
// 64 KB at d = 128, where two workgroups per CU still fit), and each wavefront
// forms its columns of J from them and its own columns of N.
//
// All products of the inverse and of J use f16 hi/lo pairs (2^-22).  A pivot
// <= 0 or a non-finite value sets a bit of the device status word.
template <int D, class TIN, bool PREP>
__global__ __launch_bounds__(kThreads, 2) void frame_kernel(PrepArgs args) {
  using T_ = typename TIN::T;
  constexpr int RT = D / 16;              // 16 x 16 tiles per row / column
  constexpr int NC = kOwnCols<RT>;        // own column tiles per wavefront
  constexpr int kTile = D * kRound;       // halves per LDS token tile
  constexpr int kTP = 20;                 // LDS pitch (floats) of a staged 16 x 16 tile
  constexpr int kStageT = RT * 16 * kTP;  // floats per sweep buffer (column p of T)
  constexpr int kSweepB = 2 * kStageT * 4 + 2 * RT * 64 * 16;  // two column buffers, two sets of RT operand tiles
  constexpr int kJB = RT * RT * 64 * 16;                     // B operand tiles of every row tile
  constexpr int kStageB = kSweepB > kJB ? kSweepB : kJB;
  constexpr int kBytes = 3 * kTile * 2 > kStageB ? 3 * kTile * 2 : kStageB;
  __shared__ __attribute__((aligned(16))) char smem[kBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  // wavefront `wave` owns column tile wave + 4 m (always, when 4 divides RT)
  auto owns = [&](int m) { return RT % 4 == 0 || wave + 4 * m < RT; };

  const int h = blockIdx.x / args.cnt;
  const int f = args.s0 + (blockIdx.x - h * args.cnt);
  const bool text = f >= args.n;
  const int U = text ? args.Nt : args.U;
  const T_* kp;
  const T_* vp;
  const float* bp;
  if (text) {
    kp = static_cast<const T_*>(args.kt) + (size_t)h * args.Nt * D;
    vp = static_cast<const T_*>(args.vt) + (size_t)h * args.Nt * D;
    bp = args.bt + (size_t)h * args.Nt;
  } else {
    const size_t fr = (size_t)h * args.T + (args.a + f);
    kp = static_cast<const T_*>(args.k) + fr * args.U * D;
    vp = static_cast<const T_*>(args.v) + fr * args.U * D;
    bp = args.beta + fr * args.U;
  }

  _Float16* sK = reinterpret_cast<_Float16*>(smem);
  _Float16* sBK = sK + kTile;
  _Float16* sBV = sBK + kTile;

  // T[m][c] = tile (c, i) of I + A, X[m][c] = tile (c, i) of B, i = wave + 4m
  f32x4 Tt[NC][RT], Xt[NC][RT];
#pragma unroll
  for (int m = 0; m < NC; ++m)
#pragma unroll
    for (int c = 0; c < RT; ++c) {
      Tt[m][c] = f32x4{0, 0, 0, 0};
      Xt[m][c] = f32x4{0, 0, 0, 0};
    }

  // ---- statistics: one load task per thread and round, 8 tokens x 8
  //      channels of K (tensor 0) or V (tensor 1), with the tokens' beta
  constexpr int CG = D / 8;
  constexpr int TASKS = 2 * (kRound / 8) * CG;  // <= 256
  const bool has_task = tid < TASKS;
  const int tensor = tid / ((kRound / 8) * CG);
  const int trem = tid - tensor * ((kRound / 8) * CG);
  const int tg = trem / CG, cg = trem - (trem / CG) * CG;
  const T_* src = tensor == 0 ? kp : vp;
  Stage8<TIN> pre;
  float pbt[8];
  auto fetch = [&](int u0) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int u = u0 + tg * 8 + s;
      const bool ok = has_task && u < U;
      pre.load(s, src + (size_t)u * D + cg * 8, ok);
      pbt[s] = ok ? bp[u] : 0.f;
    }
  };
  if (U > 0) fetch(0);
  for (int u0 = 0; u0 < U; u0 += kRound) {
    if (has_task) {
      float sc[8];  // per-token factor of the operand: beta, with raw keys also 1 / ||k||
      float rn[8];
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        rn[s] = 1.f;
        sc[s] = PREP ? sigmoid_gate(pbt[s]) : pbt[s];
      }
      if (PREP && tensor == 0) {
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          rn[s] = __builtin_amdgcn_rsqf(group_sum<CG>(pre.sumsq(s)) + kPrepEps);
          sc[s] *= rn[s];
        }
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        f16x8 pb;
#pragma unroll
        for (int s = 0; s < 8; ++s) pb[s] = (_Float16)(sc[s] * pre.get(s, c));
        *reinterpret_cast<f16x8*>((tensor == 0 ? sBK : sBV) + tile_off(cg * 8 + c, tg)) = pb;
        if (tensor == 0) {
          f16x8 pk;
#pragma unroll
          for (int s = 0; s < 8; ++s) pk[s] = (_Float16)(PREP ? pre.get(s, c) * rn[s] : pre.get(s, c));
          *reinterpret_cast<f16x8*>(sK + tile_off(cg * 8 + c, tg)) = pk;
        }
      }
    }
    lds_barrier();
    if (u0 + kRound < U) fetch(u0 + kRound);  // in flight during the MFMAs
#pragma unroll
    for (int kk = 0; kk < kRound / 32; ++kk) {
      const int grp = kk * 4 + lg;
      f16x8 bK[NC], bBK[NC];
#pragma unroll
      for (int m = 0; m < NC; ++m) {
        const int i = wave + 4 * m;
        if (owns(m)) {
          bK[m] = *reinterpret_cast<const f16x8*>(sK + tile_off(16 * i + lr, grp));
          bBK[m] = *reinterpret_cast<const f16x8*>(sBK + tile_off(16 * i + lr, grp));
        }
      }
#pragma unroll
      for (int c = 0; c < RT; ++c) {
        const f16x8 aK = *reinterpret_cast<const f16x8*>(sK + tile_off(16 * c + lr, grp));
        const f16x8 aV = *reinterpret_cast<const f16x8*>(sBV + tile_off(16 * c + lr, grp));
#pragma unroll
        for (int m = 0; m < NC; ++m) {
          if (owns(m)) {
            Tt[m][c] = mfma_f16(aK, bBK[m], Tt[m][c]);
            Xt[m][c] = mfma_f16(aV, bK[m], Xt[m][c]);
          }
        }
      }
    }
    lds_barrier();
  }

  int bad = 0;
#pragma unroll
  for (int m = 0; m < NC; ++m)
#pragma unroll
    for (int c = 0; c < RT; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (!__builtin_isfinite(Tt[m][c][e]) || !__builtin_isfinite(Xt[m][c][e])) bad |= VDA_DEV_NONFINITE;
        if (c == wave + 4 * m && 4 * lg + e == lr) Tt[m][c][e] += 1.f;  // G = I + A
      }
    }

  // ---- blocked Gauss-Jordan inverse of G, fully unrolled (tile indices
  //      constant).  Column p is staged (float32) by its owner once its pivot
  //      tile is inverted.  The step's left factors -T[j][p] Ei^T (j != p) are
  //      formed once per workgroup, spread over the wavefronts, and staged as
  //      ready f16 hi/lo A operands; after a second barrier every wavefront
  //      updates its columns from them.  The owner of column p + 1 updates
  //      the next pivot tile first and the rest of that column while it
  //      inverts the pivot, stages the column, and leaves its other column
  //      to the next step (the left factors are double-buffered for it), so
  //      that the next step's barrier waits for the inversion alone.
  float* raw = reinterpret_cast<float*>(smem);                     // 2 x RT float32 tiles
  f16x8* packs_base = reinterpret_cast<f16x8*>(raw + 2 * kStageT);  // 2 x RT operand tiles, 64 lanes each
  const f16x8 eye_hi = eye_f16(lr, lg, 0, 1.f), eye_lo = eye_f16(lr, lg, 1, 1.f);
  const f16x8 neye = eye_f16(lr, lg, -1, -1.f);  // [-I | -I]
  auto put_tile = [&](float* buf, int slot, f32x4 v) {  // tile -> row-major 16 x 16 at pitch kTP
#pragma unroll
    for (int e = 0; e < 4; ++e) buf[slot * 16 * kTP + (4 * lg + e) * kTP + lr] = v[e];
  };
  auto row_of = [&](const float* buf, int slot) {  // lane (m, g): row m, columns 4g .. 4g+3
    return *reinterpret_cast<const f32x4*>(buf + slot * 16 * kTP + lr * kTP + 4 * lg);
  };
  auto pivot_and_stage = [&](int q, int mq) {  // the owner of column q
    f32x4 y = Tt[mq][q];
    invert16(y, lr, lg, bad);  // the inverse in the same (accumulator) layout
    Tt[mq][q] = y;
    float* buf = raw + (q & 1) * kStageT;
#pragma unroll
    for (int j = 0; j < RT; ++j) put_tile(buf, j, Tt[mq][j]);  // slot q holds Ei^T
  };
  // T[j][i] += L_j T[p][i] for the own columns in `cols` (bit m: column
  // wave + 4m) and every row tile j != pp, then T[pp][i] = -Ei^T T[pp][i],
  // with the left factors L_j of step pp in pk
  auto update_cols = [&](int pp, const f16x8* pk, f16x8 neit, int cols) {
    RightF16 tpi[NC];
#pragma unroll
    for (int m = 0; m < NC; ++m)
      if ((cols >> m) & 1) tpi[m] = right_f16(Tt[m][pp]);
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      if (j == pp) continue;
      const f16x8 l = pk[j * 64 + lane];
#pragma unroll
      for (int m = 0; m < NC; ++m)
        if ((cols >> m) & 1) Tt[m][j] = mul_f16(l, tpi[m], Tt[m][j]);
    }
#pragma unroll
    for (int m = 0; m < NC; ++m)
      if ((cols >> m) & 1) Tt[m][pp] = mul_f16(neit, tpi[m], f32x4{0, 0, 0, 0});
  };
  f16x8 neit_keep;  // -Ei^T of the step whose update the pivot owner left over
  if (wave == 0) pivot_and_stage(0, 0);
#pragma unroll
  for (int p = 0; p < RT; ++p) {
    const int owner = p % 4, mo = p / 4;
    const int q = p + 1, owner1 = q % 4, mq = q / 4;
    lds_barrier();
    const float* buf = raw + (p & 1) * kStageT;
    f16x8* packs = packs_base + (p & 1) * (RT * 64);
    // left factors: -T[j][p] Ei^T = -(Ei (T[j][p])^T)^T for j = wave (mod 4);
    // the accumulator registers of Ei (T[j][p])^T are the A operand
    {
      f32x4 ei_rows;  // Ei in A-operand layout: lane (m, g) needs Ei^T[4g + e][m]
#pragma unroll
      for (int e = 0; e < 4; ++e) ei_rows[e] = buf[p * 16 * kTP + (4 * lg + e) * kTP + lr];
      const f16x8 ei_l = left_f16(ei_rows);
#pragma unroll
      for (int j = 0; j < RT; ++j)
        if (j != p && j % 4 == wave)
          packs[j * 64 + lane] = neg_f16(left_f16(mul_f16(ei_l, right_f16(row_of(buf, j)), f32x4{0, 0, 0, 0})));
    }
    const f16x8 neit_l = neg_f16(left_f16(row_of(buf, p)));  // -Ei^T
    lds_barrier();
    if (wave == owner) {  // the new column p: T[j][p] Ei^T = (-L)(-I)
#pragma unroll
      for (int j = 0; j < RT; ++j)
        if (j != p) Tt[mo][j] = mfma_f16(packs[j * 64 + lane], neye, f32x4{0, 0, 0, 0});
    }
    // the owner of column p inverted this step's pivot at step p - 1 and
    // left its other columns' update of that step until now
    if (p > 0 && wave == owner) {
      int late = 0;
#pragma unroll
      for (int m = 0; m < NC; ++m)
        if (owns(m) && wave + 4 * m != p - 1 && wave + 4 * m != p) late |= 1 << m;
      if (late) update_cols(p - 1, packs_base + ((p - 1) & 1) * (RT * 64), neit_keep, late);
    }
    int mine = 0;  // own columns other than p
#pragma unroll
    for (int m = 0; m < NC; ++m)
      if (owns(m) && wave + 4 * m != p) mine |= 1 << m;
    if (q < RT && wave == owner1) {
      // column q: the pivot tile first, then the rest of the column, whose
      // products run while the pivot is inverted; the column is then staged
      const RightF16 tq = right_f16(Tt[mq][p]);
      Tt[mq][q] = mul_f16(packs[q * 64 + lane], tq, Tt[mq][q]);
#pragma unroll
      for (int j = 0; j < RT; ++j)
        if (j != p && j != q) Tt[mq][j] = mul_f16(packs[j * 64 + lane], tq, Tt[mq][j]);
      Tt[mq][p] = mul_f16(neit_l, tq, f32x4{0, 0, 0, 0});
      pivot_and_stage(q, mq);
      neit_keep = neit_l;  // the other columns: next step
    } else {
      update_cols(p, packs, neit_l, mine);
    }
  }

  // ---- N (f16, fragment order) to the slot.  T = N^T and N is symmetric,
  //      so tile (c, i) of T is N[16c + 4g + e][16i + n] = N[16i + n][16c + 4g + e]
  //      in lane (n, g): half of the 16-byte chunk (16i + n, 2c + g/2).
  float* slot = args.frames + ((size_t)h * args.n_eff + f) * ws_slot_floats(D);
  _Float16* nf = reinterpret_cast<_Float16*>(slot);
  f16x4* jf = reinterpret_cast<f16x4*>(reinterpret_cast<char*>(slot) + 2 * D * D);
#pragma unroll
  for (int m = 0; m < NC; ++m) {
    const int i = wave + 4 * m;
    if (!owns(m)) continue;
#pragma unroll
    for (int c = 0; c < RT; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (!__builtin_isfinite(Tt[m][c][e])) bad |= VDA_DEV_NONFINITE;
      const size_t off = (size_t)ntile_chunk(D, 16 * i + lr, 2 * c + (lg >> 1)) * 8 + 4 * (lg & 1);
      *reinterpret_cast<f16x4*>(nf + off) = __builtin_convertvector(Tt[m][c], f16x4);
    }
  }

  // ---- J = B N (f16, the untransposed accumulator order: the f16x4 at
  //      (r RT + i) 64 + lane holds tile (r, i)), every row tile in one
  //      round: the owners of the columns k stage the tiles B[r][k] as ready
  //      A operands, then every wavefront forms
  //      J[r][i] = sum_k B[r][k] N[k][i] for its columns i (N[k][i] is its own
  //      tile T[k][i]).
  f16x8* bpk = reinterpret_cast<f16x8*>(smem);
  {
    lds_barrier();  // the previous readers of this memory are done
#pragma unroll
    for (int m = 0; m < NC; ++m)
      if (owns(m)) {
#pragma unroll
        for (int rr = 0; rr < RT; ++rr)
          bpk[(rr * RT + wave + 4 * m) * 64 + lane] = to_left_f16(Xt[m][rr], eye_hi, eye_lo);
      }
    lds_barrier();
#pragma unroll
    for (int m = 0; m < NC; ++m) {
      const int i = wave + 4 * m;
      if (!owns(m)) continue;
      f32x4 acc[RT];
#pragma unroll
      for (int rr = 0; rr < RT; ++rr) acc[rr] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        const RightF16 nki = right_f16(Tt[m][k]);
#pragma unroll
        for (int rr = 0; rr < RT; ++rr) acc[rr] = mul_f16(bpk[(rr * RT + k) * 64 + lane], nki, acc[rr]);
      }
#pragma unroll
      for (int rr = 0; rr < RT; ++rr) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (!__builtin_isfinite(acc[rr][e])) bad |= VDA_DEV_NONFINITE;
        jf[(rr * RT + i) * 64 + lane] = __builtin_convertvector(acc[rr], f16x4);
      }
    }
  }
  if (bad) atomicOr(args.status, bad);
}

// The SANA-WM comparator's transition in place of the factorisation: the
// batched additive update ("Video DeltaNet: A Video-Native Hybrid Attention
// for Livestream Video Generation", core-method section, paragraph 2) is
// S_t = S_bar_t (I - A'_t) + B'_t with the keys scaled by 1/sqrt(U), i.e.
// A' = A / U and B' = B / sqrt(U) (U = tokens of the slot: the frame's, or
// the text tokens).  One workgroup per slot: A's upper-triangle tiles are
// staged into LDS as the full symmetric matrix, -A / U is written over them
// as f16 in the fragment order of N (the scan adds the identity part
// itself: f16 holds -A/U to 2^-12 of its own size, while next to 1 its
// spacing would be a large part of A/U), then B is staged and rewritten in
// place as B' (f16) in the scan's accumulator order: the f16x4 at index
// (R * d/16 + ct) * 64 + l holds B'[16R + 4(l/16) + e][16ct + l%16].
template <int D>
__global__ __launch_bounds__(kThreads) void sana_kernel(PrepArgs args) {
  constexpr int RT = D / 16;
  constexpr int AP = D + 4;  // LDS pitch (floats) of A
  constexpr int BP = D + 8;  // LDS pitch (halves) of B
  constexpr int KS = D >= 32 ? D / 32 : 1;
  constexpr int LG = D >= 32 ? 4 : D / 8;
  __shared__ __attribute__((aligned(16))) float sA[D * AP];

  const int tid = threadIdx.x;
  const int h = blockIdx.x / args.cnt;
  const int f = args.s0 + (blockIdx.x - h * args.cnt);
  float* slot = args.frames + ((size_t)h * args.n_eff + f) * ws_slot_floats(D);
  const int U = f < args.n ? args.U : args.Nt;
  const float inv_u = U > 0 ? 1.f / (float)U : 0.f;
  const float inv_su = U > 0 ? 1.f / sqrtf((float)U) : 0.f;
  int bad = 0;

  // ---- A: tile (ri, cj), cj >= ri, lane l holds A[16ri + 4(l/16) + e][16cj + l%16]
  for (int i = tid; i < RT * RT * 64; i += kThreads) {
    const int l = i & 63, t = i >> 6;
    const int ri = t / RT, cj = t - ri * RT;
    if (cj < ri) continue;
    const f32x4 v = *reinterpret_cast<const f32x4*>(slot + (size_t)i * 4);
    const int c = 16 * cj + (l & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * ri + 4 * (l >> 4) + e;
      sA[r * AP + c] = v[e];
      if (cj != ri) sA[c * AP + r] = v[e];
    }
  }
  __syncthreads();
  // ---- -A / U in fragment order (chunk q holds row j, columns 8c .. 8c+7)
  f16x8* tf = reinterpret_cast<f16x8*>(slot);
  for (int q = tid; q < D * D / 8; q += kThreads) {
    const int t = q / (16 * LG);
    const int c = 4 * (t % KS) + (q / 16) % LG;
    const int j = 16 * (t / KS) + (q & 15);
    f16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = -inv_u * sA[j * AP + 8 * c + e];
      if (!__builtin_isfinite(x)) bad |= VDA_DEV_NONFINITE;
      o[e] = (_Float16)x;
    }
    tf[q] = o;
  }
  __syncthreads();
  // ---- B (row-major f16 at byte 4 d^2) -> B' = B / sqrt(U) in accumulator order, in place
  _Float16* sB = reinterpret_cast<_Float16*>(sA);
  f16x8* bm = reinterpret_cast<f16x8*>(slot + D * D);
  for (int i = tid; i < D * D / 8; i += kThreads) {
    const int r = i / (D / 8), c8 = i - r * (D / 8);
    *reinterpret_cast<f16x8*>(sB + r * BP + 8 * c8) = bm[i];
  }
  __syncthreads();
  f16x4* bo = reinterpret_cast<f16x4*>(slot + D * D);
  for (int q = tid; q < D * D / 4; q += kThreads) {
    const int l = q & 63, t = q >> 6;
    const int rt = t / RT, ct = t - rt * RT;
    const int row = 16 * rt + 4 * (l >> 4), col = 16 * ct + (l & 15);
    f16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x = inv_su * (float)sB[(row + e) * BP + col];
      if (!__builtin_isfinite(x)) bad |= VDA_DEV_NONFINITE;
      o[e] = (_Float16)x;
    }
    bo[q] = o;
  }
  if (bad) atomicOr(args.status, bad);
}

// Newton iteration for N = (I + A)^{-1} in place of the Gauss-Jordan
// inverse ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream
// Video Generation", experiments section, the weaknesses discussion: Newton
// iteration instead of the exact inverse).  G = I + A is symmetric with
// eigenvalues in [1, g], g its largest absolute row sum, so from
// X_0 = c I, c = 2 / (1 + g), the residual I - G X_k is (I - c G)^(2^k) with
// norm <= r^(2^k), r = (g - 1) / (g + 1); k is the smallest count with
// r^(2^k) <= kNsTol.  Each step is X <- X + X R with R = I - G X, i.e.
// X (2I - G X), whose residual is exactly R^2 whether or not X commutes
// with G (the left-sided X + R X needs that, and the f16 steps break it at
// the 1e-3 level, where the iteration then stalls).  X and R are written to
// LDS transposed, so the columns of X (B operands of G X) and of R (B
// operands of X R) are rows there.  The A operand of X R takes the rows of
// X^T, i.e. the columns of X: X is symmetric up to rounding, and that
// difference enters the residual only multiplied by R.
// Precision: the steps before the last form G X from f16 G and X (the
// residual then stalls near 1e-3); the last step forms G X from f16 hi/lo
// pairs of both (float32 accuracy), which squares that residual away.  X is
// kept in float32 accumulators throughout; R X uses f16 R and X (R is small).
// One workgroup per matrix; a wavefront owns D/NWV rows of every product.
constexpr float kNsTol = 1e-6f;

template <int D>
struct NsShape {
  static constexpr int NWV = D / 16;                // wavefronts: one 16-row tile each
  static constexpr int NTH = 64 * NWV;
  static constexpr int RT = D / 16;                 // 16-row tiles of the matrix
  static constexpr int RTW = RT / NWV;              // row tiles per wavefront
  static constexpr int KS = D >= 32 ? D / 32 : 1;   // MFMA k-steps (D = 16: one, zero padded)
  static constexpr int AP = D + 4;                  // LDS pitch (floats) of the A staging
  static constexpr int XP = D + 8;                  // LDS pitch (halves) of X and R
  static constexpr int LDS = D * AP * 4 > 2 * D * XP * 2 ? D * AP * 4 : 2 * D * XP * 2;
};

template <int D>
__global__ __launch_bounds__(NsShape<D>::NTH, 2) void ns_kernel(PrepArgs args) {
  using NS = NsShape<D>;
  constexpr int RT = NS::RT, RTW = NS::RTW, KS = NS::KS, AP = NS::AP, XP = NS::XP;
  __shared__ __attribute__((aligned(16))) float lds[NS::LDS / 4];
  __shared__ float sMax[NS::NWV];
  float* sA = lds;
  _Float16* sXh = reinterpret_cast<_Float16*>(lds);  // X (f16 hi)
  _Float16* sXl = sXh + D * XP;                      // X (f16 lo), or R

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int h = blockIdx.x / args.cnt;
  const int f = args.s0 + (blockIdx.x - h * args.cnt);
  float* slot = args.frames + ((size_t)h * args.n_eff + f) * ws_slot_floats(D);
  int bad = 0;

  // ---- A (upper-triangle tiles, accumulator layout) -> LDS, full symmetric
  for (int i = tid; i < RT * RT * 64; i += NS::NTH) {
    const int l = i & 63, t = i >> 6;
    const int ri = t / RT, cj = t - ri * RT;
    if (cj < ri) continue;
    const f32x4 v = *reinterpret_cast<const f32x4*>(slot + (size_t)i * 4);
    const int c = 16 * cj + (l & 15);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 16 * ri + 4 * (l >> 4) + e;
      sA[r * AP + c] = v[e];
      if (cj != ri) sA[c * AP + r] = v[e];
    }
  }
  __syncthreads();
  // ---- this wavefront's rows of G = I + A as A operands (hi/lo); row sums of |G|
  f16x8 gh[RTW][KS], gl[RTW][KS];
  float rs[RTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const int m = 16 * (wave * RTW + rt) + lr;
    rs[rt] = 0.f;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int k0 = 32 * kk + 8 * lg;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float gv = k0 < D ? (m == k0 + e ? 1.f : 0.f) + sA[m * AP + k0 + e] : 0.f;
        const _Float16 hi = (_Float16)gv;
        gh[rt][kk][e] = hi;
        gl[rt][kk][e] = (_Float16)(gv - (float)hi);
        rs[rt] += fabsf(gv);
      }
    }
    rs[rt] += __shfl_xor(rs[rt], 16, 64);
    rs[rt] += __shfl_xor(rs[rt], 32, 64);
  }
  float gmax = 0.f;
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) gmax = fmaxf(gmax, rs[rt]);
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) gmax = fmaxf(gmax, __shfl_xor(gmax, off, 64));
  if (lane == 0) sMax[wave] = gmax;
  __syncthreads();  // also: every wavefront is done with the A staging
  gmax = sMax[0];
#pragma unroll
  for (int w = 1; w < NS::NWV; ++w) gmax = fmaxf(gmax, sMax[w]);
  if (!__builtin_isfinite(gmax)) bad |= VDA_DEV_NONFINITE;
  const float r = (gmax - 1.f) / (gmax + 1.f);
  int k = 0;
  for (float pw = r; pw > kNsTol && k < 64; pw *= pw) ++k;
  const float c0 = 2.f / (1.f + gmax);

  // ---- X in float32 accumulators: x[rt][ct][e] = X[16(wave RTW + rt) + 4lg + e][16ct + lr]
  f32x4 x[RTW][RT];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int ct = 0; ct < RT; ++ct)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        x[rt][ct][e] = (16 * (wave * RTW + rt) + 4 * lg + e == 16 * ct + lr) ? c0 : 0.f;
  // X^T = X to LDS: the 4 rows of a lane land as 4 consecutive halves of row 16ct + lr
  auto put_x = [&](bool with_lo) {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < RT; ++ct) {
        f16x4 hi, lo;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hi[e] = (_Float16)x[rt][ct][e];
          lo[e] = (_Float16)(x[rt][ct][e] - (float)hi[e]);
        }
        const int at = (16 * ct + lr) * XP + 16 * (wave * RTW + rt) + 4 * lg;
        *reinterpret_cast<f16x4*>(sXh + at) = hi;
        if (with_lo) *reinterpret_cast<f16x4*>(sXl + at) = lo;
      }
  };
  // B operand: row n = 16ct + lr (= column n), k = 32kk + 8lg .. +7
  auto brow = [&](const _Float16* buf, int ct, int kk) {
    const int k0 = 32 * kk + 8 * lg;
    f16x8 v;
    if (k0 < D) {
      v = *reinterpret_cast<const f16x8*>(buf + (16 * ct + lr) * XP + k0);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = (_Float16)0.f;
    }
    return v;
  };
  put_x(k == 1);
  __syncthreads();
  for (int it = 0; it < k; ++it) {
    const bool last = it == k - 1;
    // Y = G X; R = I - Y
    f32x4 y[RTW][RT];
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < RT; ++ct) y[rt][ct] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int ct = 0; ct < RT; ++ct)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const f16x8 xb = brow(sXh, ct, kk);
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) y[rt][ct] = mfma_f16(gh[rt][kk], xb, y[rt][ct]);
        if (last) {
          const f16x8 xl = brow(sXl, ct, kk);
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt) {
            y[rt][ct] = mfma_f16(gh[rt][kk], xl, y[rt][ct]);
            y[rt][ct] = mfma_f16(gl[rt][kk], xb, y[rt][ct]);
          }
        }
      }
    __syncthreads();  // X lo is read before R takes its place
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
      for (int ct = 0; ct < RT; ++ct) {
        f16x4 rv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float id = (16 * (wave * RTW + rt) + 4 * lg + e == 16 * ct + lr) ? 1.f : 0.f;
          rv[e] = (_Float16)(id - y[rt][ct][e]);
        }
        *reinterpret_cast<f16x4*>(sXl + (16 * ct + lr) * XP + 16 * (wave * RTW + rt) + 4 * lg) = rv;  // R^T
      }
    __syncthreads();
    // X <- X + X R: A operand = this wavefront's rows of X^T, B operand = rows of R^T
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      f16x8 xa[RTW];
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
        const int k0 = 32 * kk + 8 * lg;
        if (k0 < D) {
          xa[rt] = *reinterpret_cast<const f16x8*>(sXh + (16 * (wave * RTW + rt) + lr) * XP + k0);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) xa[rt][e] = (_Float16)0.f;
        }
      }
#pragma unroll
      for (int ct = 0; ct < RT; ++ct) {
        const f16x8 rb = brow(sXl, ct, kk);
#pragma unroll
        for (int rt = 0; rt < RTW; ++rt) x[rt][ct] = mfma_f16(xa[rt], rb, x[rt][ct]);
      }
    }
    __syncthreads();
    if (!last) {
      put_x(it + 1 == k - 1);
      __syncthreads();
    }
  }

  // ---- N = X -> workspace as f16 in fragment order; a tile covers column
  //      16ct + lr, rows 16R + 4lg + e: half of chunk (16ct + lr, 2R + lg/2)
  _Float16* nf = reinterpret_cast<_Float16*>(slot);
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt)
#pragma unroll
    for (int ct = 0; ct < RT; ++ct) {
      const int R = wave * RTW + rt;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (!__builtin_isfinite(x[rt][ct][e])) bad |= VDA_DEV_NONFINITE;
      const size_t off = (size_t)ntile_chunk(D, 16 * ct + lr, 2 * R + (lg >> 1)) * 8 + 4 * (lg & 1);
      *reinterpret_cast<f16x4*>(nf + off) = __builtin_convertvector(x[rt][ct], f16x4);
    }
  if (bad) atomicOr(args.status, bad);
}

__global__ void clear_status_kernel(int* status) { *status = 0; }
__global__ void copy_status_kernel(const int* src, int32_t* dst) { *dst = *src; }

void launch_copy_status(const int* src, int32_t* dst, hipStream_t stream) {
  hipLaunchKernelGGL(copy_status_kernel, dim3(1), dim3(1), 0, stream, src, dst);
}

int launch_stats(const PrepArgs& a, int d, bool in_f32, hipStream_t stream) {
  if (a.H == 0 || a.cnt == 0) return 0;
  dim3 grid((unsigned)(a.H * a.cnt)), block(kThreads);
#define VDA_STATS(DD)                                                                 \
  if (d == DD) {                                                                      \
    if (in_f32 && a.prep)                                                             \
      hipLaunchKernelGGL((stats_kernel<DD, InF32, true>), grid, block, 0, stream, a); \
    else if (in_f32)                                                                  \
      hipLaunchKernelGGL((stats_kernel<DD, InF32, false>), grid, block, 0, stream, a); \
    else if (a.prep)                                                                  \
      hipLaunchKernelGGL((stats_kernel<DD, InBF16, true>), grid, block, 0, stream, a); \
    else                                                                              \
      hipLaunchKernelGGL((stats_kernel<DD, InBF16, false>), grid, block, 0, stream, a); \
    return 0;                                                                         \
  }
  VDA_STATS(16) VDA_STATS(32) VDA_STATS(64) VDA_STATS(128)
#undef VDA_STATS
  return -1;
}

int launch_frame(const PrepArgs& a, int d, bool in_f32, hipStream_t stream) {
  if (a.H == 0 || a.cnt == 0) return 0;
  dim3 grid((unsigned)(a.H * a.cnt)), block(kThreads);
#define VDA_FRAME(DD)                                                                 \
  if (d == DD) {                                                                      \
    if (in_f32 && a.prep)                                                             \
      hipLaunchKernelGGL((frame_kernel<DD, InF32, true>), grid, block, 0, stream, a); \
    else if (in_f32)                                                                  \
      hipLaunchKernelGGL((frame_kernel<DD, InF32, false>), grid, block, 0, stream, a); \
    else if (a.prep)                                                                  \
      hipLaunchKernelGGL((frame_kernel<DD, InBF16, true>), grid, block, 0, stream, a); \
    else                                                                              \
      hipLaunchKernelGGL((frame_kernel<DD, InBF16, false>), grid, block, 0, stream, a); \
    return 0;                                                                         \
  }
  VDA_FRAME(16) VDA_FRAME(32) VDA_FRAME(64) VDA_FRAME(128)
#undef VDA_FRAME
  return -1;
}

int launch_ns(const PrepArgs& a, int d, hipStream_t stream) {
  if (a.H == 0 || a.cnt == 0) return 0;
  dim3 grid((unsigned)(a.H * a.cnt));
#define VDA_NS(DD)                                                                    \
  if (d == DD) {                                                                      \
    hipLaunchKernelGGL((ns_kernel<DD>), grid, dim3(NsShape<DD>::NTH), 0, stream, a);  \
    return 0;                                                                         \
  }
  VDA_NS(16) VDA_NS(32) VDA_NS(64) VDA_NS(128)
#undef VDA_NS
  return -1;
}

int launch_sana(const PrepArgs& a, int d, hipStream_t stream) {
  if (a.H == 0 || a.cnt == 0) return 0;
  dim3 grid((unsigned)(a.H * a.cnt)), block(kThreads);
#define VDA_SANA(DD)                                                                  \
  if (d == DD) {                                                                      \
    hipLaunchKernelGGL((sana_kernel<DD>), grid, block, 0, stream, a);                 \
    return 0;                                                                         \
  }
  VDA_SANA(16) VDA_SANA(32) VDA_SANA(64) VDA_SANA(128)
#undef VDA_SANA
  return -1;
}

void launch_clear_status(int* status, hipStream_t stream) {
  hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(1), 0, stream, status);
}

}  // namespace vda
