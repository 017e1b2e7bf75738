// Window-excluding bidirectional readout.
//
// For a scanned frame t of chunk c ("Video DeltaNet: A Video-Native Hybrid
// Attention for Livestream Video Generation", core-method section,
// paragraph 1, and method-steps section, step (5)):
//
//   O_t = Q_t W_t^T,   W_t = S^f_{F(c)} Diag(b_f) + S^r_{R(c)} Diag(b_r),
//   b_f = prod_{r=ws}^{t} alpha_r,   b_r = prod_{r=t}^{we} alpha_r,
//
// i.e. the forward state that ends before the softmax window and the reverse
// state that starts after it, each carried to frame t through the decay of
// the excluded frames.  The two reads are merged into one d x d operand W_t
// per frame, so the token GEMM runs once.  With no window exclusion the
// readout is O_t = Q_t (S^f_t)^T.  Anchor frames get zero rows.
//
// One workgroup per (head, frame), ordered so that the frames of one head
// run on one XCD.  Wavefront w owns value-channel tiles
// w, w+4, ... (for d = 128: the two tiles of wavefront w interleave channels
// 32w .. 32w+31 so that each lane stores 8 consecutive channels of a token
// with one 16-byte store) and keeps its rows of W_t in registers as bf16
// hi/lo pairs;
// 128-token tiles of Q are staged in LDS with one coalesced pass (the next
// tile's loads are issued before the current tile's MFMAs) and each
// wavefront computes O^T = W Q^T on MFMA (2 products per tile for bf16 Q,
// 3 for float32 Q split hi/lo), accumulating in float32.
//
// The gated launch adds the epilogue of the linear branch (same page,
// method-steps section, step (5): the read is RMS-normalised, then gated by a
// sigmoid; core-method section, paragraph 1: the linear branch is normalised
// before its gate):  y_c = o_c / sqrt(mean_c o_c^2 + eps) * w_c * sigmoid(g_c)
// over the d value channels of each token.  A wavefront holds a quarter of a
// token's channels, so each 64-token tile takes two passes over its MFMAs:
// the first leaves per-token partial sums of squares in LDS, and after one
// extra barrier the second recomputes the products (cheaper than keeping
// them, which would cost a workgroup per CU) and stores the normalised,
// gated outputs.  The tile's gate logits are loaded before its products.
#include "vda_common.h"
#include "vda_kernels.h"

namespace vda {

namespace {

constexpr int kQT = 128;  // tokens per LDS tile (64 in the gated launch)

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <int OUT>
struct OutT;
template <>
struct OutT<VDA_F32> {
  static __device__ __forceinline__ void store4(void* base, size_t idx, f32x4 v) {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + idx) = make_float4(v[0], v[1], v[2], v[3]);
  }
  static __device__ __forceinline__ void store8(void* base, size_t idx, f32x4 v, f32x4 w) {
    store4(base, idx, v);
    store4(base, idx + 4, w);
  }
  static constexpr int bytes = 4;
};
template <>
struct OutT<VDA_BF16> {
  static __device__ __forceinline__ void store4(void* base, size_t idx, f32x4 v) {
    bf16x4 b = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *reinterpret_cast<bf16x4*>(static_cast<u16*>(base) + idx) = b;
  }
  static __device__ __forceinline__ void store8(void* base, size_t idx, f32x4 v, f32x4 w) {
    bf16x8 b = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3],
                (__bf16)w[0], (__bf16)w[1], (__bf16)w[2], (__bf16)w[3]};
    *reinterpret_cast<bf16x8*>(static_cast<u16*>(base) + idx) = b;
  }
  static constexpr int bytes = 2;
};
template <>
struct OutT<VDA_F16> {
  static __device__ __forceinline__ void store4(void* base, size_t idx, f32x4 v) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    h4 p = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    *reinterpret_cast<h4*>(static_cast<_Float16*>(base) + idx) = p;
  }
  static __device__ __forceinline__ void store8(void* base, size_t idx, f32x4 v, f32x4 w) {
    typedef _Float16 h8 __attribute__((ext_vector_type(8)));
    h8 p = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3],
            (_Float16)w[0], (_Float16)w[1], (_Float16)w[2], (_Float16)w[3]};
    *reinterpret_cast<h8*>(static_cast<_Float16*>(base) + idx) = p;
  }
  static constexpr int bytes = 2;
};

// Q operand (eight consecutive channels of one token) from the LDS tile.
template <class TIN>
struct QFrag;
template <>
struct QFrag<InBF16> {
  bf16x8 hi;
  __device__ __forceinline__ void load(const char* row, int k0, bool in) {
    if (in) {
      hi = *reinterpret_cast<const bf16x8*>(row + 2 * k0);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) hi[e] = bits_to_bf16(0);
    }
  }
};
template <>
struct QFrag<InF32> {
  bf16x8 hi, lo;
  __device__ __forceinline__ void load(const char* row, int k0, bool in) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = in ? reinterpret_cast<const float*>(row)[k0 + e] : 0.f;
      __bf16 h, l;
      split_bf16(x, h, l);
      hi[e] = h;
      lo[e] = l;
    }
  }
};

// N consecutive gate logits of one token, kept as loaded until used.
template <class TIN, int N>
struct GateRaw;
template <>
struct GateRaw<InBF16, 8> {
  uint4 r;
  __device__ __forceinline__ void load(const void* base, size_t idx) {
    r = *reinterpret_cast<const uint4*>(static_cast<const u16*>(base) + idx);
  }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t w = (e >> 1) == 0 ? r.x : (e >> 1) == 1 ? r.y : (e >> 1) == 2 ? r.z : r.w;
    return bf16_bits_to_f32((e & 1) ? (w >> 16) : (w & 0xffffu));
  }
};
template <>
struct GateRaw<InBF16, 4> {
  uint2 r;
  __device__ __forceinline__ void load(const void* base, size_t idx) {
    r = *reinterpret_cast<const uint2*>(static_cast<const u16*>(base) + idx);
  }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t w = (e >> 1) == 0 ? r.x : r.y;
    return bf16_bits_to_f32((e & 1) ? (w >> 16) : (w & 0xffffu));
  }
};
template <>
struct GateRaw<InF32, 8> {
  float4 r[2];
  __device__ __forceinline__ void load(const void* base, size_t idx) {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
    r[0] = p[0];
    r[1] = p[1];
  }
  __device__ __forceinline__ float get(int e) const {
    const float4 v = r[e >> 2];
    return (e & 3) == 0 ? v.x : (e & 3) == 1 ? v.y : (e & 3) == 2 ? v.z : v.w;
  }
};
template <>
struct GateRaw<InF32, 4> {
  float4 r;
  __device__ __forceinline__ void load(const void* base, size_t idx) {
    r = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + idx);
  }
  __device__ __forceinline__ float get(int e) const { return e == 0 ? r.x : e == 1 ? r.y : e == 2 ? r.z : r.w; }
};

// Sum of squares of the 16 bytes of one token row chunk (8 bf16 or 4 float32).
template <class TIN>
__device__ __forceinline__ float chunk_sumsq(uint4 w) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if constexpr (TIN::bytes == 2) {
      const float lo = __uint_as_float(u[q] << 16), hi = __uint_as_float(u[q] & 0xffff0000u);
      ss = fmaf(lo, lo, fmaf(hi, hi, ss));
    } else {
      const float x = __uint_as_float(u[q]);
      ss = fmaf(x, x, ss);
    }
  }
  return ss;
}

// Sum of v over the four 16-lane rows of the wavefront, in every lane
// (permlane32_swap pairs rows (0, 2) and (1, 3), permlane16_swap then (0, 1)).
__device__ __forceinline__ float sum_rows4(float v) {
  const unsigned b = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  const float s = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const unsigned c = __float_as_uint(s);
  const auto q = __builtin_amdgcn_permlane16_swap(c, c, false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

}  // namespace

template <int D, class TIN, int OUT, bool GATED, bool PREP>
__global__ __launch_bounds__(kThreads, GATED ? 3 : 2) void readout_kernel(ReadArgs a) {
  using T = typename TIN::T;
  constexpr int VT = D / 16;                         // value-channel tiles
  constexpr int NVT = (VT + 3) / 4;                  // tiles per wavefront
  constexpr int KS = D / 32 > 0 ? D / 32 : 1;        // MFMA k-steps
  constexpr int QT = GATED ? 64 : kQT;               // tokens per LDS tile
  constexpr int PITCH = D * TIN::bytes + 16;         // LDS bytes per token row
  constexpr int CH = D * TIN::bytes / 16;            // 16-byte chunks per token row
  constexpr int PER = (QT * CH + kThreads - 1) / kThreads;  // chunks per thread per tile
  // d = 128: the two tiles of wavefront w interleave its 32 value channels so
  // that a lane's outputs of one token are 8 consecutive channels
  constexpr bool kPair = VT == 8;
  auto chan = [](int w, int i, int r) {
    return kPair ? 32 * w + 8 * (r >> 2) + 4 * i + (r & 3) : 16 * (w + 4 * i) + r;
  };
  __shared__ __attribute__((aligned(16))) char sQ[QT * PITCH];
  __shared__ float sBf[D], sBr[D];
  __shared__ float sRq[PREP ? QT : 1];  // raw q: 1 / ||q|| of the tile's tokens

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  // the frames of one head run on one XCD: its L2 keeps the states that
  // the frames of a chunk and its neighbours share
  const int L = xcd_block(blockIdx.x, gridDim.x);
  const int h = L / a.T;
  const int t = L - h * a.T;
  const size_t frame_off = ((size_t)h * a.T + t) * (size_t)a.U * D;

  if (t < a.a || t >= a.T - a.a) {  // anchor frame: zero rows
    constexpr int per16 = 16 / OutT<OUT>::bytes;
    const size_t n16 = (size_t)a.U * D / per16;
    uint4* o = reinterpret_cast<uint4*>(static_cast<char*>(a.out) + frame_off * OutT<OUT>::bytes);
    for (size_t i = tid; i < n16; i += kThreads) o[i] = make_uint4(0, 0, 0, 0);
    return;
  }

  // ---- first Q tile in flight while the states and bridges are read
  const T* qh = static_cast<const T*>(a.q) + frame_off;
  uint4 pre[PER];
  auto fetch = [&](int u0) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + j * kThreads;
      const int r = i / CH, ch = i - r * CH;
      pre[j] = (i < QT * CH && u0 + r < a.U)
                   ? reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(qh + (size_t)(u0 + r) * D))[ch]
                   : make_uint4(0, 0, 0, 0);
    }
  };
  fetch(0);

  // ---- states and bridges for this frame; without the epilogue this lane's
  // entries of the two states are loaded first, so that their latency
  // overlaps the bridges' (the bridges' alpha loads and the states' otherwise
  // make two round trips to memory in a row before the first product; the
  // gated launch, at three workgroups per CU, has no registers to hold them)
  const int f = t - a.a;
  const float* sf;
  const float* sr = nullptr;
  float4 rf[NVT][KS][2], rr[NVT][KS][2];
  auto load_states = [&]() {
    if constexpr (GATED) return;
#pragma unroll
    for (int i = 0; i < NVT; ++i) {
      const int vt = wave + 4 * i;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int k0 = 32 * kk + 8 * lg;
        if (vt < VT && k0 < D) {
          const size_t idx = (size_t)chan(wave, i, lr) * D + k0;
          rf[i][kk][0] = *reinterpret_cast<const float4*>(sf + idx);
          rf[i][kk][1] = *reinterpret_cast<const float4*>(sf + idx + 4);
          if (sr) {
            rr[i][kk][0] = *reinterpret_cast<const float4*>(sr + idx);
            rr[i][kk][1] = *reinterpret_cast<const float4*>(sr + idx + 4);
          }
        }
      }
    }
  };
  const float* alpha_h = a.alpha + (size_t)h * a.T * D;
  if (a.w >= 0) {
    const ChunkWindow cw = chunk_window(frame_chunk_of(t, a.a, a.n, a.P), a.C, a.w, a.P, a.a, a.n);
    const int ws = cw.ws, we = cw.we;
    sf = a.sf + ((size_t)h * a.count + cw.F) * D * D;
    sr = a.sr + ((size_t)h * a.count + cw.R) * D * D;
    load_states();  // in flight while the bridges are formed
    // thread k < D: forward bridge of channel k; D <= k < 2D: reverse bridge
    for (int k2 = tid; k2 < 2 * D; k2 += kThreads) {
      const bool rev = k2 >= D;
      const int k = rev ? k2 - D : k2;
      const int r0 = rev ? t : ws, r1 = rev ? we : t;  // inclusive frame range
      float prod = 1.f;
      if (a.bridge) {
        for (int rb = r0; rb <= r1; rb += 16) {  // 16 loads in flight per pass
          float v[16];
#pragma unroll
          for (int j = 0; j < 16; ++j) v[j] = (rb + j <= r1) ? alpha_h[(size_t)(rb + j) * D + k] : 1.f;
          if constexpr (PREP) {  // alpha given as logits
#pragma unroll
            for (int j = 0; j < 16; ++j) v[j] = (rb + j <= r1) ? sigmoid_gate(v[j]) : 1.f;
          }
#pragma unroll
          for (int j = 0; j < 16; ++j) prod *= v[j];
        }
      }
      (rev ? sBr : sBf)[k] = prod;
    }
  } else {
    sf = a.sf + ((size_t)h * a.count + f + 1) * D * D;
    load_states();
    for (int k = tid; k < D; k += kThreads) {
      sBf[k] = 1.f;
      sBr[k] = 0.f;
    }
  }
  lds_barrier();

  // ---- W rows of this wavefront's value tiles, bf16 hi/lo, A-operand layout
  bf16x8 wh[NVT][KS], wl[NVT][KS];
#pragma unroll
  for (int i = 0; i < NVT; ++i) {
    const int vt = wave + 4 * i;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int k0 = 32 * kk + 8 * lg;
      float x[8];
      if (vt < VT && k0 < D) {
        const size_t idx = (size_t)chan(wave, i, lr) * D + k0;
        const float4 f0 = GATED ? *reinterpret_cast<const float4*>(sf + idx) : rf[i][kk][0];
        const float4 f1 = GATED ? *reinterpret_cast<const float4*>(sf + idx + 4) : rf[i][kk][1];
        x[0] = f0.x * sBf[k0]; x[1] = f0.y * sBf[k0 + 1]; x[2] = f0.z * sBf[k0 + 2]; x[3] = f0.w * sBf[k0 + 3];
        x[4] = f1.x * sBf[k0 + 4]; x[5] = f1.y * sBf[k0 + 5]; x[6] = f1.z * sBf[k0 + 6]; x[7] = f1.w * sBf[k0 + 7];
        if (sr) {
          const float4 r0 = GATED ? *reinterpret_cast<const float4*>(sr + idx) : rr[i][kk][0];
          const float4 r1 = GATED ? *reinterpret_cast<const float4*>(sr + idx + 4) : rr[i][kk][1];
          x[0] = fmaf(r0.x, sBr[k0], x[0]); x[1] = fmaf(r0.y, sBr[k0 + 1], x[1]);
          x[2] = fmaf(r0.z, sBr[k0 + 2], x[2]); x[3] = fmaf(r0.w, sBr[k0 + 3], x[3]);
          x[4] = fmaf(r1.x, sBr[k0 + 4], x[4]); x[5] = fmaf(r1.y, sBr[k0 + 5], x[5]);
          x[6] = fmaf(r1.z, sBr[k0 + 6], x[6]); x[7] = fmaf(r1.w, sBr[k0 + 7], x[7]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 hh, ll;
        split_bf16(x[e], hh, ll);
        wh[i][kk][e] = hh;
        wl[i][kk][e] = ll;
      }
    }
  }

  // ---- gated epilogue: RMSNorm weights of this lane's channels
  constexpr int GN = kPair ? 8 : 4;  // consecutive channels per gate / output access
  constexpr int NG = kPair ? 1 : NVT;
  constexpr int NSUB = QT / 16;
  float nw[NVT][4];
  if constexpr (GATED) {
#pragma unroll
    for (int i = 0; i < NVT; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        nw[i][e] = (wave + 4 * i < VT) ? a.normw[(size_t)h * D + chan(wave, i, 4 * lg + e)] : 0.f;
  }
  __shared__ float sSq[GATED ? 4 * QT : 1];  // per-wavefront partial sums of squares per token

  // One tile with the epilogue: the per-token sums of squares of the four
  // wavefronts meet in LDS, then y = o * rsqrt(mean o^2 + eps) * w *
  // sigmoid(g) is stored.
  auto gated_tile = [&](int u0) {
    GateRaw<TIN, GN> graw[NSUB][NG];
    // gate logits of the tile first: they arrive during the products
#pragma unroll
    for (int st = 0; st < NSUB; ++st) {
      const int u = u0 + 16 * st + lr;
      if (wave < VT && u < a.U) {
        if constexpr (kPair) {
          graw[st][0].load(a.gate, frame_off + (size_t)u * D + 32 * wave + 8 * lg);
        } else {
#pragma unroll
          for (int i = 0; i < NVT; ++i)
            if (wave + 4 * i < VT) graw[st][i].load(a.gate, frame_off + (size_t)u * D + 16 * (wave + 4 * i) + 4 * lg);
        }
      }
    }
    auto products = [&](int st, f32x4 (&acc)[NVT]) {
      const int ul = 16 * st + lr;
#pragma unroll
      for (int i = 0; i < NVT; ++i) acc[i] = f32x4{0, 0, 0, 0};
      if (wave < VT && u0 + 16 * st < a.U) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const int k0 = 32 * kk + 8 * lg;
          QFrag<TIN> qf;
          qf.load(sQ + ul * PITCH, k0, k0 < D);
#pragma unroll
          for (int i = 0; i < NVT; ++i) {
            if (wave + 4 * i < VT) {
              acc[i] = mfma_bf16(wh[i][kk], qf.hi, acc[i]);
              acc[i] = mfma_bf16(wl[i][kk], qf.hi, acc[i]);
              if constexpr (TIN::bytes == 4) acc[i] = mfma_bf16(wh[i][kk], qf.lo, acc[i]);
            }
          }
        }
        if constexpr (PREP) {
          const float rq = sRq[ul];
#pragma unroll
          for (int i = 0; i < NVT; ++i) acc[i] *= rq;
        }
      }
    };
    // pass 1: per-token sums of squares of this wavefront's channels
#pragma unroll
    for (int st = 0; st < NSUB; ++st) {
      f32x4 acc[NVT];
      products(st, acc);
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < NVT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) ss = fmaf(acc[i][e], acc[i][e], ss);
      ss = sum_rows4(ss);
      if (lg == 0) sSq[wave * QT + 16 * st + lr] = ss;
    }
    lds_barrier();
    // pass 2: the products again, normalised, gated and stored
    if (wave < VT) {
#pragma unroll
      for (int st = 0; st < NSUB; ++st) {
        const int ul = 16 * st + lr;
        const int u = u0 + ul;
        f32x4 acc[NVT];
        products(st, acc);
        if (u >= a.U) continue;
        const float tot = sSq[ul] + sSq[QT + ul] + sSq[2 * QT + ul] + sSq[3 * QT + ul];
        const float rs = __builtin_amdgcn_rsqf(tot * (1.f / D) + a.eps);
        f32x4 y[NVT];
#pragma unroll
        for (int i = 0; i < NVT; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float g = kPair ? graw[st][0].get(4 * i + e) : graw[st][i].get(e);
            y[i][e] = acc[i][e] * rs * nw[i][e] * sigmoid_gate(g);
          }
        if constexpr (kPair) {
          OutT<OUT>::store8(a.out, frame_off + (size_t)u * D + 32 * wave + 8 * lg, y[0], y[1]);
        } else {
#pragma unroll
          for (int i = 0; i < NVT; ++i) {
            const int vt = wave + 4 * i;
            if (vt < VT) OutT<OUT>::store4(a.out, frame_off + (size_t)u * D + 16 * vt + 4 * lg, y[i]);
          }
        }
      }
    }
  };

  // ---- token tiles: the next tile's loads are in flight during the MFMAs
  for (int u0 = 0; u0 < a.U; u0 += QT) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = tid + j * kThreads;
      if (i < QT * CH) {
        const int r = i / CH, ch = i - r * CH;
        *reinterpret_cast<uint4*>(sQ + r * PITCH + 16 * ch) = pre[j];
      }
    }
    if constexpr (PREP) {  // raw q: the output of token u is scaled by 1 / ||q_u|| (o = S q / ||q||)
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int i = tid + j * kThreads;
        const float ss = group_sum<CH>(chunk_sumsq<TIN>(pre[j]));
        const int r = i / CH;
        if (i < QT * CH && i - r * CH == 0) sRq[r] = __builtin_amdgcn_rsqf(ss + kPrepEps);
      }
    }
    lds_barrier();
    if (u0 + QT < a.U) fetch(u0 + QT);
    if constexpr (GATED) {
      gated_tile(u0);
    } else if (wave < VT) {
      const int nsub = (a.U - u0) >= QT ? QT / 16 : (a.U - u0 + 15) / 16;
      for (int st = 0; st < nsub; ++st) {
        const int ul = 16 * st + lr;  // token of this lane's operand column
        f32x4 acc[NVT];
#pragma unroll
        for (int i = 0; i < NVT; ++i) acc[i] = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const int k0 = 32 * kk + 8 * lg;
          QFrag<TIN> qf;
          qf.load(sQ + ul * PITCH, k0, k0 < D);
#pragma unroll
          for (int i = 0; i < NVT; ++i) {
            if (wave + 4 * i < VT) {
              acc[i] = mfma_bf16(wh[i][kk], qf.hi, acc[i]);
              acc[i] = mfma_bf16(wl[i][kk], qf.hi, acc[i]);
              if constexpr (TIN::bytes == 4) acc[i] = mfma_bf16(wh[i][kk], qf.lo, acc[i]);
            }
          }
        }
        const int u = u0 + ul;
        if constexpr (PREP) {
          const float rq = sRq[ul];
#pragma unroll
          for (int i = 0; i < NVT; ++i) acc[i] *= rq;
        }
        if (u < a.U) {
          if constexpr (kPair) {
            OutT<OUT>::store8(a.out, frame_off + (size_t)u * D + 32 * wave + 8 * lg, acc[0], acc[1]);
          } else {
#pragma unroll
            for (int i = 0; i < NVT; ++i) {
              const int vt = wave + 4 * i;
              if (vt < VT) OutT<OUT>::store4(a.out, frame_off + (size_t)u * D + 16 * vt + 4 * lg, acc[i]);
            }
          }
        }
      }
    }
    lds_barrier();
  }
}

// Index maps on the device: thread c < C writes row c, thread C + t < C + T
// the chunk of frame t.
__global__ void index_map_kernel(int C, int T, int w, int P, int a, int n, int32_t* rows, int32_t* fc) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < C) {
    const ChunkWindow cw = chunk_window(i, C, w, P, a, n);
    int32_t* r = rows + 7 * (size_t)i;
    r[0] = i;
    r[1] = cw.lo;
    r[2] = cw.hi;
    r[3] = cw.ws;
    r[4] = cw.we;
    r[5] = cw.F;
    r[6] = cw.R;
  } else if (i < C + T) {
    fc[i - C] = frame_chunk_of(i - C, a, n, P);
  }
}

void launch_index_map(int C, int T, int w, int P, int a, int n, int32_t* rows, int32_t* frame_chunk,
                      hipStream_t stream) {
  const int total = C + T;
  if (total <= 0) return;
  hipLaunchKernelGGL(index_map_kernel, dim3((total + 255) / 256), dim3(256), 0, stream, C, T, w, P, a, n, rows,
                     frame_chunk);
}

template <bool GATED>
static int launch_readout_impl(const ReadArgs& a, int d, int in_dtype, int out_dtype, hipStream_t stream) {
  if (a.H == 0 || a.T == 0) return 0;
  dim3 grid((unsigned)(a.H * a.T)), block(kThreads);
#define VDA_RD3(DD, TI, OO)                                                                         \
  if (out_dtype == OO) {                                                                            \
    if (a.prep)                                                                                     \
      hipLaunchKernelGGL((readout_kernel<DD, TI, OO, GATED, true>), grid, block, 0, stream, a);     \
    else                                                                                            \
      hipLaunchKernelGGL((readout_kernel<DD, TI, OO, GATED, false>), grid, block, 0, stream, a);    \
    return 0;                                                                                       \
  }
#define VDA_RD(DD)                                                                 \
  if (d == DD) {                                                                   \
    if (in_dtype == VDA_F32) {                                                     \
      VDA_RD3(DD, InF32, VDA_F32) VDA_RD3(DD, InF32, VDA_BF16) VDA_RD3(DD, InF32, VDA_F16) \
    } else {                                                                       \
      VDA_RD3(DD, InBF16, VDA_F32) VDA_RD3(DD, InBF16, VDA_BF16) VDA_RD3(DD, InBF16, VDA_F16) \
    }                                                                              \
    return -1;                                                                     \
  }
  VDA_RD(16) VDA_RD(32) VDA_RD(64) VDA_RD(128)
#undef VDA_RD
#undef VDA_RD3
  return -1;
}

int launch_readout(const ReadArgs& a, int d, int in_dtype, int out_dtype, hipStream_t stream) {
  return launch_readout_impl<false>(a, d, in_dtype, out_dtype, stream);
}

int launch_readout_gated(const ReadArgs& a, int d, int in_dtype, int out_dtype, hipStream_t stream) {
  return launch_readout_impl<true>(a, d, in_dtype, out_dtype, stream);
}

}  // namespace vda
