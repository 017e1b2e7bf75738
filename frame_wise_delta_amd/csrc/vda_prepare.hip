// Frame statistics and factorisation of the VDA frame write, as two kernels.
//
// stats_kernel: for every (head, frame) one workgroup computes, over the
// frame's U tokens,
//   A = K^T Diag(beta) K  and  B = V^T Diag(beta) K
// ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
// Generation", method-steps section, step (3)) on MFMA with float32
// accumulation, and stores B (row-major) and the upper-triangle tiles of A
// (accumulator layout, in the place N will take) in the frame's workspace
// slot.  K, V rows are streamed from HBM in 64-token rounds, converted
// to f16 (beta*K is rounded once to f16) and written channel-major into LDS
// so that an MFMA operand lane reads eight consecutive tokens of one channel
// with a single 16-byte LDS load.  The 16-byte token groups of each LDS row
// are XOR-swizzled so that both the transposing writes and the operand reads
// are free of bank conflicts.  The next round's global loads are issued
// before the current round's MFMAs.
//
// gj_kernel: one wavefront per frame inverts G = I + A in registers with a
// blocked Gauss-Jordan sweep (16x16 blocks on MFMA, scalar 16x16 pivot-block
// inverses) and overwrites A with N = G^{-1}, rounded to f16, in the MFMA
// fragment order the scan consumes.  G is symmetric positive definite
// (eigenvalues >= 1), so no pivoting is needed.  Running the latency-bound
// sweep as single-wavefront workgroups, apart from the bandwidth-bound
// statistics, lets every SIMD work on its own matrices without barriers.
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

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// bf16 pair with v ~ hi + lo: hi is v truncated to bf16 (exact upper half
// of the float32 word), lo = v - hi (exact) rounded to bf16, so hi + lo
// holds v to about 2^-16 relative.
__device__ __forceinline__ void split4(f32x4 v, bf16x4& hi, bf16x4& lo) {
  uint32_t w[4];
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w[e] = __float_as_uint(v[e]);
    r[e] = v[e] - __uint_as_float(w[e] & 0xffff0000u);
  }
  uint2 h;
  h.x = __builtin_amdgcn_perm(w[1], w[0], 0x07060302u);  // upper halves of w0 (low) and w1 (high)
  h.y = __builtin_amdgcn_perm(w[3], w[2], 0x07060302u);
  hi = __builtin_bit_cast(bf16x4, h);
  lo = __builtin_convertvector(r, bf16x4);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 neg8(bf16x8 a) {
  uint4 u = __builtin_bit_cast(uint4, a);
  u.x ^= 0x80008000u; u.y ^= 0x80008000u; u.z ^= 0x80008000u; u.w ^= 0x80008000u;
  return __builtin_bit_cast(bf16x8, u);
}

// Index of the upper-triangle tile pair {i, j}, i <= j, of a RT x RT grid.
__host__ __device__ constexpr int upair(int RT, int i, int j) { return i * RT - i * (i - 1) / 2 + (j - i); }

// 16x16 float32 transposes through LDS, for accumulator-layout tiles (lane
// (n, g) holds Z[4g + e][n]).  put stores Z^T row-major; get returns the
// accumulator layout of Z^T.  The 20-float pitch keeps both conflict-free.
constexpr int kXP = 20;
__device__ __forceinline__ void tr_put(float* buf, f32x4 v, int n, int g) {
  *reinterpret_cast<f32x4*>(buf + n * kXP + 4 * g) = v;
}
__device__ __forceinline__ f32x4 tr_get(const float* buf, int n, int g) {
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = buf[(4 * g + e) * kXP + n];
  return r;
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

// One wavefront inverts one G = I + A.  G is symmetric, so only the pairs
// {i, j}, i <= j, of 16x16 tiles are kept, each once, in MFMA accumulators
// (lane (n, g) holds rows 4g .. 4g+3 of column n of the tile).  In-place
// Gauss-Jordan over the blocks P processed so far keeps the working matrix M
// symmetric within P and within the rest Q, and antisymmetric between them
// (M[i][j] = -M[j][i]^T for i in P, j in Q), so either tile of a pair gives
// the other.  A pair {i, j}, i < j, is held as M[i][j] until step j and as
// M[j][i] from then on: at step p every pair {j, p} is held as M[p][j], the
// row strip R_j of the pivot (the pairs {j, p}, j < p, are transposed through
// LDS at the start of step p).  Step p:
//   E = M[p][p] -> E^{-1}, scalar Gauss-Jordan, four columns per lane;
//   r'_j = E^{-1} R_j on MFMA, the new M[p][j] (the new column strip follows
//          by the symmetry above and is never formed);
//   every other pair, held as M[x][y]: M[x][y] -= M[x][p] r'_y, where the
//          operand M[x][p] comes from R_x (= +R_x^T for x > p and -R_x^T
//          for x < p).
// An accumulator tile Z used as the MFMA A operand is Z^T and as the B operand
// Z itself, so every product above reads the tiles in place.  Products use
// bf16 hi/lo splits of both factors; the K = 32 MFMA forms (a_hi + a_lo) b in
// one instruction by pairing the hi and lo halves of one factor with two
// copies of one half of the other, so a four-term product takes two MFMAs.
// The pivot block is read as E^T (equal to E) and E^{-1} is used as its own
// transpose.  A pivot <= 0 or a non-finite value sets a bit of the device
// status word.
template <int D>
__global__ __launch_bounds__(64, 2) void gj_kernel(PrepArgs args) {
  constexpr int RT = D / 16;
  constexpr int NPR = RT * (RT + 1) / 2;
  constexpr int NB = RT > 1 ? RT - 1 : 1;  // transpose buffers
  __shared__ __attribute__((aligned(16))) float sT[NB][16 * kXP];

  const int lane = threadIdx.x;
  const int n = lane & 15, g = lane >> 4;
  const int h = blockIdx.x / args.cnt;
  const int f = args.s0 + (blockIdx.x - h * args.cnt);
  float* slot = args.frames + ((size_t)h * args.n_eff + f) * ws_slot_floats(D);
  int bad = 0;

  // ---- G = I + A from the upper-triangle tiles of A (accumulator layout)
  f32x4 G[NPR];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = i; j < RT; ++j)
      G[upair(RT, i, j)] = *reinterpret_cast<const f32x4*>(slot + ((size_t)(i * RT + j) * 64 + lane) * 4);
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) G[upair(RT, i, i)][e] += (4 * g + e == n) ? 1.0f : 0.0f;

  // ---- blocked Gauss-Jordan, fully unrolled (every tile index is constant)
#pragma unroll
  for (int p = 0; p < RT; ++p) {
    if (p > 0) {  // pairs {j, p}, j < p: M[j][p] -> M[p][j] = -M[j][p]^T
#pragma unroll
      for (int j = 0; j < p; ++j) tr_put(sT[j], G[upair(RT, j, p)], n, g);
      lds_barrier();
#pragma unroll
      for (int j = 0; j < p; ++j) G[upair(RT, j, p)] = -tr_get(sT[j], n, g);
      lds_barrier();
    }
    f32x4 y = G[upair(RT, p, p)];
    invert16(y, n, g, bad);
    G[upair(RT, p, p)] = y;
    bf16x8 e_hh, e_ll;  // A operands [Einv_hi | Einv_hi], [Einv_lo | Einv_lo]
    {
      bf16x4 hi, lo;
      split4(y, hi, lo);
      e_hh = cat8(hi, hi);
      e_ll = cat8(lo, lo);
    }
    bf16x8 xr[RT];  // [R_hi | R_lo] of the row strip
#pragma unroll
    for (int j = 0; j < RT; ++j)
      if (j != p) {
        bf16x4 hi, lo;
        split4(G[upair(RT, j < p ? j : p, j < p ? p : j)], hi, lo);
        xr[j] = cat8(hi, lo);
      }
    // r'_j, then every pair held as M[x][j]: for j > p the pairs {a, j}
    // (held as M[a][j]), for j < p the pairs {j, b}, b < p (held as M[b][j])
#pragma unroll
    for (int j = 0; j < RT; ++j)
      if (j != p) {
        f32x4 r = mfma_bf16(e_hh, xr[j], f32x4{0, 0, 0, 0});
        r = mfma_bf16(e_ll, xr[j], r);
        G[upair(RT, j < p ? j : p, j < p ? p : j)] = r;
        bf16x4 hi, lo;
        split4(r, hi, lo);
        const bf16x8 b_hh = cat8(hi, hi), b_ll = cat8(lo, lo);  // B operands of r'_j
        const bf16x8 n_hh = neg8(b_hh), n_ll = neg8(b_ll);
#pragma unroll
        for (int x = 0; x < RT; ++x) {
          const bool held = j > p ? (x <= j && x != p) : (x >= j && x < p);
          if (!held) continue;
          const int t = upair(RT, x < j ? x : j, x < j ? j : x);
          // M[x][j] -= M[x][p] r'_j with M[x][p] = -R_x^T (x < p), +R_x^T (x > p)
          f32x4 acc = G[t];
          acc = mfma_bf16(xr[x], x > p ? n_hh : b_hh, acc);
          acc = mfma_bf16(xr[x], x > p ? n_ll : b_ll, acc);
          G[t] = acc;
        }
      }
  }

  // ---- N = G^{-1} -> workspace as f16 in fragment order.  Pair
  //      {i, j}, i < j, is held as N[j][i]; N[i][j] is its transpose.  An
  //      accumulator tile N[x][y] covers column 16y + n, rows 16x + 4g + e,
  //      i.e. half of the 16-byte chunk (16y + n, 2x + g/2).
  _Float16* nf = reinterpret_cast<_Float16*>(slot);
  auto put = [&](f32x4 v, int x, int yy) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (!__builtin_isfinite(v[e])) bad |= VDA_DEV_NONFINITE;
    const size_t off = (size_t)ntile_chunk(D, 16 * yy + n, 2 * x + (g >> 1)) * 8 + 4 * (g & 1);
    *reinterpret_cast<f16x4*>(nf + off) = __builtin_convertvector(v, f16x4);
  };
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    put(G[upair(RT, j, j)], j, j);
#pragma unroll
    for (int i = 0; i < j; ++i) {
      put(G[upair(RT, i, j)], j, i);
      tr_put(sT[i], G[upair(RT, i, j)], n, g);
    }
    if (j > 0) {
      lds_barrier();
#pragma unroll
      for (int i = 0; i < j; ++i) put(tr_get(sT[i], n, g), i, j);
      lds_barrier();
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

int launch_gj(const PrepArgs& a, int d, hipStream_t stream) {
  if (a.H == 0 || a.cnt == 0) return 0;
  dim3 grid((unsigned)(a.H * a.cnt)), block(64);
#define VDA_GJ(DD)                                                                    \
  if (d == DD) {                                                                      \
    hipLaunchKernelGGL((gj_kernel<DD>), grid, block, 0, stream, a);                   \
    return 0;                                                                         \
  }
  VDA_GJ(16) VDA_GJ(32) VDA_GJ(64) VDA_GJ(128)
#undef VDA_GJ
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
