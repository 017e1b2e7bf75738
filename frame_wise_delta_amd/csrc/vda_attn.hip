// Softmax branch of the hybrid attention: exact softmax attention of every
// query token over its visible keys ("Video DeltaNet: A Video-Native Hybrid
// Attention for Livestream Video Generation", core-method section, paragraph
// 1, and method-steps section, step (1)):
//
//   query frames of chunk c   see the frames of chunks c-w .. c+w (clipped),
//                             the two anchor frames and the text tokens;
//   anchor frames (0, T-1)    see every frame and the text tokens;
//
//   o = softmax(q K^T * scale) V  over those keys.
//
// Flash-attention style: one 512-thread workgroup per 256 query tokens of
// one query block (a chunk's frames, or one anchor frame), eight wavefronts
// of 32 queries, so that every key tile is fetched and staged once for 256
// queries.  Keys stream through LDS in 64-key tiles, segment by segment
// (window frames, anchor frames, text), rotating through three LDS buffers
// with one barrier per tile; the next two tiles' loads are in flight, in two
// register sets, during the current tile's work.  The second wavefront of
// each SIMD runs one step behind the first (it accumulates the previous tile
// before it scores the current one), so that one wavefront's exponentials
// overlap the other's MFMAs.  The scores are formed transposed,
// S^T = K Q^T (16x16x32 bf16 MFMA), so that a wavefront's accumulator lane
// holds four consecutive keys of one query; two such tiles make the B
// operand of a 16x16x32 MFMA.  The output is accumulated transposed as well,
// O^T += V^T P^T on f16 operands (P rounded once; V given as f16, or bf16
// converted while it is staged in LDS), with V^T read with the LDS
// transposing load in the same key order; the softmax denominators come out
// of the same MFMAs (an all-ones row block in place of V^T).  The softmax is online (running max and
// sum per query, in float32, base 2).
#include <type_traits>

#include "vda_common.h"
#include "vda_kernels.h"

namespace vda {

namespace {

constexpr int kQB = 256;  // queries per workgroup
constexpr int kAT = 512;  // threads per workgroup: eight wavefronts of 32 queries
constexpr int kKT = 64;   // keys per LDS tile

typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;


// max over the four 16-lane rows (lanes n, n+16, n+32, n+48), in
// every lane: permlane32_swap pairs rows (0, 2) and (1, 3), permlane16_swap
// then rows (0, 1).
__device__ __forceinline__ float rows4_max(float v) {
  const unsigned b = __float_as_uint(v);
  const auto p = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  const float s = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  const unsigned c = __float_as_uint(s);
  const auto q = __builtin_amdgcn_permlane16_swap(c, c, false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

// One key tile's P (f16) for a wavefront's two 16-query tiles: v[kp][qt]
// holds keys 32 kp + 4g + e, then 32 kp + 16 + 4g + e (lane group g).
struct PTile {
  f16x8 v[2][2];
};

template <int OUT>
__device__ __forceinline__ void store_out4(void* base, size_t idx, f32x4 v) {
  if constexpr (OUT == VDA_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + idx) = make_float4(v[0], v[1], v[2], v[3]);
  } else if constexpr (OUT == VDA_BF16) {
    bf16x4 b = {(__bf16)v[0], (__bf16)v[1], (__bf16)v[2], (__bf16)v[3]};
    *reinterpret_cast<bf16x4*>(static_cast<u16*>(base) + idx) = b;
  } else {
    f16x4 h = {(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    *reinterpret_cast<f16x4*>(static_cast<_Float16*>(base) + idx) = h;
  }
}

}  // namespace

// Query blocks of one head, in this order: [anchor frame 0], the C chunks,
// [anchor frame T-1]; block b has nq(b) query tokens starting at token
// q0(b) of the head and ceil(nq / kQB) workgroups.
template <int D, int OUT, bool VF16>
__global__ __launch_bounds__(kAT, 1) void attn_kernel(AttnArgs a) {
  static_assert(D % 32 == 0 && D <= 128, "head size must be 32, 64 or 128");
  constexpr int KS = D / 32;   // k-steps of the score product
  constexpr int DT = D / 16;   // 16-wide output tiles
  constexpr int KP = D + 16;   // LDS row pitch (halves): rows 32 bytes apart modulo 256
  constexpr int CPR = D / 8;   // 16-byte chunks per key row
  constexpr int NCH = kKT * CPR;               // 16-byte chunks per tile (K and V each)
  constexpr int LPT = (NCH + kAT - 1) / kAT;   // chunks per thread per tile
  // three tile buffers: tile j lives in buffer j % 3 (see the loop below)
  __shared__ __attribute__((aligned(16))) u16 sK[3 * kKT * KP];
  __shared__ __attribute__((aligned(16))) _Float16 sV[3 * kKT * KP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 15, lg = lane >> 4;

  // ---- which head, query block and 256-query tile
  int L = xcd_block(blockIdx.x, gridDim.x);
  const int h = L / a.tiles_per_head;
  L -= h * a.tiles_per_head;
  const int ta = a.anchor_tiles;  // tiles per anchor frame (0 without anchors)
  const int tc = a.chunk_tiles;   // tiles per chunk
  int qb, tile;                   // query block (-1: first anchor, C: last anchor), tile in it
  if (L < ta) {
    qb = -1;
    tile = L;
  } else if (L < ta + a.C * tc) {
    qb = (L - ta) / tc;
    tile = L - ta - qb * tc;
  } else {
    qb = a.C;
    tile = L - ta - a.C * tc;
  }
  const bool anchor_q = qb < 0 || qb >= a.C;
  const int qf0 = qb < 0 ? 0 : (anchor_q ? a.T - 1 : a.a + a.P * qb);  // first query frame
  const int nq = (anchor_q ? 1 : a.P) * a.U;                           // query tokens in the block
  const int q0 = qf0 * a.U + tile * kQB;                                 // first query token of the tile
  const int nq_tile = nq - tile * kQB < kQB ? nq - tile * kQB : kQB;

  // ---- key segments: [start, end) tokens of the head's video keys, then text
  int seg_s[3], seg_e[3], nseg = 0;
  if (anchor_q) {
    seg_s[0] = 0;
    seg_e[0] = a.T * a.U;
    nseg = 1;
  } else {
    const ChunkWindow cw = chunk_window(qb, a.C, a.w, a.P, a.a, a.T - 2 * a.a);
    seg_s[0] = cw.ws * a.U;
    seg_e[0] = (cw.we + 1) * a.U;
    nseg = 1;
    if (a.a) {
      seg_s[1] = 0;
      seg_e[1] = a.U;
      seg_s[2] = (a.T - 1) * a.U;
      seg_e[2] = a.T * a.U;
      nseg = 3;
    }
  }
  int ntiles = 0;
  for (int s = 0; s < nseg; ++s) ntiles += (seg_e[s] - seg_s[s] + kKT - 1) / kKT;
  const int text_tiles = (a.Nt + kKT - 1) / kKT;
  const int all_tiles = ntiles + text_tiles;

  const size_t hoff = (size_t)h * a.T * a.U * D;
  const u16* qh = static_cast<const u16*>(a.q) + hoff;
  const u16* kh = static_cast<const u16*>(a.k) + hoff;
  const u16* vh = static_cast<const u16*>(a.v) + hoff;
  const u16* kth = static_cast<const u16*>(a.kt) + (size_t)h * a.Nt * D;
  const u16* vth = static_cast<const u16*>(a.vt) + (size_t)h * a.Nt * D;

  // ---- Q fragments (B operand of S^T = K Q^T): lane (n, g) holds query n's
  // channels 32 kk + 8g .. +7, for its wavefront's two 16-query tiles
  bf16x8 qf[2][KS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qi = wave * 32 + qt * 16 + ln;
    const bool ok = qi < nq_tile;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const uint4 w = ok ? *reinterpret_cast<const uint4*>(qh + (size_t)(q0 + qi) * D + 32 * kk + 8 * lg)
                         : make_uint4(0, 0, 0, 0);
      qf[qt][kk] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // ---- key tile j: its source rows and valid count
  auto tile_src = [&](int j, const u16*& kb, const u16*& vb, int& n) {
    if (j >= ntiles) {  // text
      const int t0 = (j - ntiles) * kKT;
      kb = kth + (size_t)t0 * D;
      vb = vth + (size_t)t0 * D;
      n = a.Nt - t0 < kKT ? a.Nt - t0 : kKT;
      return;
    }
    for (int s = 0; s < nseg; ++s) {
      const int nt = (seg_e[s] - seg_s[s] + kKT - 1) / kKT;
      if (j < nt) {
        const int t0 = seg_s[s] + j * kKT;
        kb = kh + (size_t)t0 * D;
        vb = vh + (size_t)t0 * D;
        n = seg_e[s] - t0 < kKT ? seg_e[s] - t0 : kKT;
        return;
      }
      j -= nt;
    }
    kb = kh;
    vb = vh;
    n = 0;
  };

  uint4 pk[2][LPT], pv[2][LPT];  // two register sets: tiles j and j + 1 in flight
  // this thread's 16-byte chunks of a key tile: row c / CPR, channels 8 (c % CPR) ..
  // (the same offsets for every tile; rows are contiguous within a segment)
  int coff[LPT], crow[LPT], loff[LPT];  // global (elements) and LDS (halves) offsets
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int c0 = tid + i * kAT;
    const int c = c0 < NCH ? c0 : 0;  // threads past the tile's chunks (d = 32) stay idle
    crow[i] = c / CPR;
    coff[i] = crow[i] * D + 8 * (c - crow[i] * CPR);
    loff[i] = crow[i] * KP + 8 * (c - crow[i] * CPR);
  }
  // chunk slot i of this thread exists (always for d >= 64)
  auto chunk_live = [&](int i) { return NCH % kAT == 0 || tid + i * kAT < NCH; };
  auto fetch = [&](int j, auto set) {
    constexpr int S = decltype(set)::value;
    const u16* kb;
    const u16* vb;
    int n;
    tile_src(j, kb, vb, n);
    if (n == kKT) {  // a full tile (every tile but a segment's last): no masks
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        if (!chunk_live(i)) continue;
        pk[S][i] = *reinterpret_cast<const uint4*>(kb + coff[i]);
        pv[S][i] = *reinterpret_cast<const uint4*>(vb + coff[i]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        if (!chunk_live(i)) continue;
        const bool ok = crow[i] < n;
        pk[S][i] = ok ? *reinterpret_cast<const uint4*>(kb + coff[i]) : make_uint4(0, 0, 0, 0);
        pv[S][i] = ok ? *reinterpret_cast<const uint4*>(vb + coff[i]) : make_uint4(0, 0, 0, 0);
      }
    }
    return n;
  };

  f32x4 o[2][DT];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[qt][dt] = f32x4{0, 0, 0, 0};
  float m_run[2] = {-INFINITY, -INFINITY};
  // row sums of P on the MFMA: an all-ones A operand makes every row of the
  // product the sum over the keys (every lane of a query holds it)
  f32x4 lsum[2] = {f32x4{0, 0, 0, 0}, f32x4{0, 0, 0, 0}};
  f16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (_Float16)1.0f;
  const float sc = a.scale * 1.4426950408889634f;  // scale to base-2 units

  // V^T fragment addressing (transposing load): lane j of 16-lane block g
  // reads key row 4g + (j >> 2) of the 16-key sub-tile, channels
  // 16 dt + 4 (j & 3) .. +3
  const int vrow = 4 * lg + (ln >> 2), vcol = 4 * (ln & 3);

  // S^T = K Q^T for tile buffer `buf`, masked past n_tile keys, then the
  // online softmax: P (f16) into p, O and the row sums rescaled when a
  // query's reference point moves
  auto scores = [&](int buf, int n_tile) {
    PTile p;
    const u16* kb = sK + buf * (kKT * KP);
    f32x4 s[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt][0] = f32x4{0, 0, 0, 0};
      s[kt][1] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kb + (16 * kt + ln) * KP + 32 * kk + 8 * lg));
        s[kt][0] = mfma_bf16(kf, qf[0][kk], s[kt][0]);
        s[kt][1] = mfma_bf16(kf, qf[1][kk], s[kt][1]);
      }
    }
    // lane (n, g) holds keys 16 kt + 4g + e of query n.  Scores stay
    // unscaled; the running max is kept in scaled base-2 units.
    if (n_tile < kKT) {  // last tile of a segment: keys past its end get no weight
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (16 * kt + 4 * lg + e >= n_tile) s[kt][0][e] = s[kt][1][e] = -INFINITY;
    }
    // p[kp][qt]: keys 32 kp + 4g + e, then 32 kp + 16 + 4g + e
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[kt][qt][e]);
      mx = rows4_max(mx) * sc;
      // The reference point m_run moves only when a score exceeds it by more
      // than 8 (base 2), so the weights stay below 2^8 (exact enough in f16)
      // and O is rescaled only on the rare tiles where some query's
      // reference moves (always on the first tile, where m_run = -inf).
      const bool move = mx > m_run[qt] + 8.f;
      const float m_new = move ? mx : m_run[qt];
      if (__builtin_amdgcn_ballot_w64(move)) {
        const float corr = __builtin_amdgcn_exp2f(m_run[qt] - m_new);  // 0 when m_run = -inf, 1 when kept
        lsum[qt] *= corr;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[qt][dt] *= corr;
        m_run[qt] = m_new;
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          p.v[kt >> 1][qt][4 * (kt & 1) + e] = (_Float16)__builtin_amdgcn_exp2f(fmaf(s[kt][qt][e], sc, -m_new));
    }
    return p;
  };
  // O^T += V^T P^T on 16x16x32 MFMA for tile buffer `buf`: the k order of a
  // 32-key pair is (16-key sub-tile 2kp, keys 4g .. 4g+3; sub-tile 2kp+1,
  // keys 4g .. 4g+3) in lane group g, the same for the V^T operand (two
  // transposing loads) and for P (two score accumulators)
  auto accumulate = [&](int buf, const PTile& p) {
    const _Float16* vb = sV + buf * (kKT * KP);
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const _Float16* src = vb + (32 * kp + vrow) * KP + 16 * dt + vcol;
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)src);
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(src + 16 * KP));
        const f16x8 vf = __builtin_bit_cast(f16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        o[0][dt] = mfma_f16(vf, p.v[kp][0], o[0][dt]);
        o[1][dt] = mfma_f16(vf, p.v[kp][1], o[1][dt]);
      }
      lsum[0] = mfma_f16(ones, p.v[kp][0], lsum[0]);
      lsum[1] = mfma_f16(ones, p.v[kp][1], lsum[1]);
    }
  };

  // Tiles alternate between the two register sets (set j % 2 holds tile j
  // until it is staged, then receives tile j + 2) and rotate through three
  // LDS buffers (tile j in buffer j % 3), with one barrier per tile.  The
  // wavefronts 0-3 run each tile as scores, softmax, accumulate; the
  // wavefronts 4-7 (the other wavefront on each SIMD) accumulate the
  // previous tile first, then take this tile's scores and softmax, keeping
  // its P for the next step.  So while one wavefront of a SIMD computes
  // exponentials the other one issues MFMAs.  Buffer j % 3 is written at
  // step j, read at steps j (both halves) and j + 1 (the second half), and
  // written again only at step j + 3, after the barrier of step j + 2.
  int n_t[2] = {0, 0};
  if (all_tiles > 0) n_t[0] = fetch(0, std::integral_constant<int, 0>{});
  if (all_tiles > 1) n_t[1] = fetch(1, std::integral_constant<int, 1>{});
  auto tile_step = [&](int j, auto set, auto lag_c, PTile& p_prev) {
    constexpr int S = decltype(set)::value;
    constexpr bool lag = decltype(lag_c)::value;
    const int buf = j % 3;
    // ---- stage tile j: K as loaded, V converted to f16
    u16* kdst = sK + buf * (kKT * KP);
    _Float16* vdst = sV + buf * (kKT * KP);
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      if (!chunk_live(i)) continue;
      *reinterpret_cast<uint4*>(kdst + loff[i]) = pk[S][i];
      if constexpr (VF16) {
        *reinterpret_cast<uint4*>(vdst + loff[i]) = pv[S][i];
      } else {  // bf16 V -> f16
        const uint32_t u[4] = {pv[S][i].x, pv[S][i].y, pv[S][i].z, pv[S][i].w};
        f16x8 hv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          hv[2 * e] = (_Float16)__uint_as_float(u[e] << 16);
          hv[2 * e + 1] = (_Float16)__uint_as_float(u[e] & 0xffff0000u);
        }
        *reinterpret_cast<f16x8*>(vdst + loff[i]) = hv;
      }
    }
    const int n_tile = n_t[S];
    lds_barrier();
    if (j + 2 < all_tiles) n_t[S] = fetch(j + 2, set);
    if constexpr (!lag) {
      accumulate(buf, scores(buf, n_tile));
    } else {
      if (j > 0) accumulate(buf == 0 ? 2 : buf - 1, p_prev);
      p_prev = scores(buf, n_tile);
    }
  };
  auto run = [&](auto lag_c) {
    PTile p_prev;
    for (int j = 0; j < all_tiles; j += 2) {
      tile_step(j, std::integral_constant<int, 0>{}, lag_c, p_prev);
      if (j + 1 < all_tiles) tile_step(j + 1, std::integral_constant<int, 1>{}, lag_c, p_prev);
    }
    if constexpr (decltype(lag_c)::value)
      if (all_tiles > 0) accumulate((all_tiles - 1) % 3, p_prev);
  };
  if (__builtin_amdgcn_readfirstlane(wave) >= 4)
    run(std::true_type{});
  else
    run(std::false_type{});

  // ---- O = O^T / l: lane (n, g) holds channels 16 dt + 4g + e of query n
  const size_t obase = (size_t)h * a.T * a.U * D;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qi = wave * 32 + qt * 16 + ln;
    if (qi >= nq_tile) continue;
    const float inv = lsum[qt][0] > 0.f ? 1.f / lsum[qt][0] : 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) store_out4<OUT>(a.out, obase + (size_t)(q0 + qi) * D + 16 * dt + 4 * lg, o[qt][dt] * inv);
  }
}

template <bool VF16>
static int launch_attn_v(const AttnArgs& a, int d, int out_dtype, hipStream_t stream) {
  dim3 grid((unsigned)(a.H * a.tiles_per_head)), block(kAT);
#define VDA_AT(DD)                                                                                         \
  if (d == DD) {                                                                                           \
    if (out_dtype == VDA_F32)                                                                              \
      hipLaunchKernelGGL((attn_kernel<DD, VDA_F32, VF16>), grid, block, 0, stream, a);                     \
    else if (out_dtype == VDA_BF16)                                                                        \
      hipLaunchKernelGGL((attn_kernel<DD, VDA_BF16, VF16>), grid, block, 0, stream, a);                    \
    else                                                                                                   \
      hipLaunchKernelGGL((attn_kernel<DD, VDA_F16, VF16>), grid, block, 0, stream, a);                     \
    return 0;                                                                                              \
  }
  VDA_AT(32) VDA_AT(64) VDA_AT(128)
#undef VDA_AT
  return -1;
}

int launch_attn(const AttnArgs& a, int d, int out_dtype, hipStream_t stream) {
  if (a.H == 0 || a.tiles_per_head == 0) return 0;
  return a.v_f16 ? launch_attn_v<true>(a, d, out_dtype, stream) : launch_attn_v<false>(a, d, out_dtype, stream);
}

}  // namespace vda
