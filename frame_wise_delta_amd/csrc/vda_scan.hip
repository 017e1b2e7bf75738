// Forward / reverse VDA scan: the only sequential part of the path.
//
//   S_t = (S_{t-1} Diag(alpha_t) + B_t) N_t = (S_{t-1} Diag(alpha_t)) N_t + J_t,
//   N_t = (I + A_t)^{-1},  J_t = B_t N_t
//
// ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
// Generation", core-method section, paragraph 2: closed-form frame write;
// method-steps section, step (4): both scans start from the text state.)
//
// The d_v rows of S evolve independently (row i: s_t = (s_{t-1} * alpha_t) N_t
// + j_t), so one (head, direction) chain is split over d/32 workgroups of
// 32 rows each (16 for d = 16); the row blocks of a head are mapped to one
// XCD so that they share that XCD's L2 copy of N_t.  A workgroup runs d/16
// wavefronts, one per 16-column tile of its 32 x d slice of S, and keeps
// the slice in the wavefronts' float32 accumulators, transposed: the
// product is taken as S^T <- N X^T (N is symmetric), so that accumulator
// lane (n, g) of column tile c holds S[n][16c + 4g .. 16c + 4g + 3] of one
// row tile.  Per frame each wavefront forms its part of X = S Diag(alpha)
// in registers (alpha is per column, so a lane needs four values), splits
// it into an f16 hi/lo pair and writes it to LDS (row-major, 16-byte pieces
// swizzled by row so that the operand reads are free of bank conflicts); after one
// barrier every wavefront reads the rows of X as the B operand (eight
// consecutive columns per lane) and runs X_hi N + X_lo N on MFMA for its
// column tile, the accumulators starting from J_t.  X is double-buffered
// in LDS, so one barrier per frame orders both its writes and its reads.
// N and J_t are stored by the prepare kernel as f16: N in MFMA fragment
// order (16-byte pieces of eight consecutive entries of a row, by 16-row
// tile and k-slice: what the A operand of N X^T takes directly), J_t in the
// accumulator order of the untransposed product, which an MFMA with the
// identity turns into this one.  The comparators'
// slots hold B_t (the Newton comparator, added into X before the product)
// or B' (SANA-WM, added after it) instead of J_t.
// Frames are prefetched several steps ahead into registers, their loads
// issued part by part between the k-steps of the current step's MFMAs, and
// the barrier waits for LDS traffic only, so the global loads stay in
// flight across it; a step is then bound by its own chain (X through LDS,
// the barrier, the products of the two wavefronts sharing each SIMD).
//
// The same kernel also runs the scan at chunk level (method-steps section,
// step (4): S_out = S_in M_chunk + J_chunk), in two launches:
//  * compose (compose_kernel): the frame write is the affine map
//    S -> S M_t + J_t with M_t = Diag(alpha_t) N_t and J_t = B_t N_t, so
//    running the frame step over a chunk's frames on the stacked 2d x d
//    state [Y; X] from [I; 0] (B zero on the Y rows) leaves Y = M_c and
//    X = J_c.  Every (head, chunk, direction) is an independent chain of P
//    steps, so all of them run at once; the reverse direction takes the
//    chunk's frames last first.  M_c is stored as f16 in the fragment order
//    of N (column j's k-slices, since M_c is not symmetric) and J_c as f16 in
//    accumulator order: the f16x4 at index (R * d/16 + ct) * 64 + l holds
//    J_c[16R + 4(l/16) + e][16ct + l%16].
//  * chunk scan: C steps of S <- S M_c + J_c, the product on the same MFMA
//    path as a frame step (S^T <- M_c^T X^T: M_c's stored columns are the
//    rows of M_c^T the A operand needs, X = S as an f16 hi/lo pair) with
//    the accumulators starting from J_c; the state is recorded after every
//    chunk, which is where the windowed readout needs it.
#include <type_traits>

#include "vda_common.h"
#include "vda_kernels.h"

namespace vda {

namespace {

// Two 16 x 16 f16 tiles held in accumulator order (lane (n, g): rows
// 4g .. 4g+3 of column n), one in each half of an f16x8, are transposed
// into float32 accumulator order exactly by one 16x16x32 MFMA each: the
// pair as the A operand (tile 0 in k-slots 8g .. 8g+3, tile 1 in
// 8g+4 .. 8g+7) times the identity placed in the slots of the wanted tile
// (eye_k32).  It is the same MFMA shape as the products that then
// accumulate onto the result, so every accumulator a product reads comes
// from an MFMA of its own shape.
__device__ __forceinline__ f16x8 eye_k32(int lr, int lg, int half) {
  f16x8 e8;
#pragma unroll
  for (int e = 0; e < 8; ++e) e8[e] = (_Float16)(e / 4 == half && 4 * lg + (e & 3) == lr ? 1.f : 0.f);
  return e8;
}
__device__ __forceinline__ f32x4 transpose_tile(f16x8 pair, f16x8 eye_half) {
  return mfma_f16(pair, eye_half, f32x4{0, 0, 0, 0});
}

template <int D>
struct ScanShape {
  static constexpr int ROWS = D < 32 ? D : 32;          // state rows per workgroup
  static constexpr int RTS = ROWS / 16;                 // 16-row tiles per workgroup
  static constexpr int NW = D / 16;                     // wavefronts = 16-column tiles
  static constexpr int NT = 64 * NW;                    // threads
  static constexpr int KS = D >= 32 ? D / 32 : 1;       // MFMA k-steps (D = 16: one, zero padded)
  static constexpr int XP = D;                          // LDS row pitch of X (halves), see x_off
  static constexpr int NQ = ROWS / 16;                  // J / B registers per lane (one per row tile)
  static constexpr int LG = D >= 32 ? 4 : D / 8;        // k-chunk groups per fragment-order block
  static constexpr int PD = D >= 128 ? 3 : (D >= 64 ? 4 : 2);  // frames prefetched ahead
};

// Offset (halves) of X[row][col] in an LDS buffer of X: unpadded rows whose
// 16-byte pieces (eight columns) are XOR-swizzled by the row.  A step's
// 16-byte operand reads (rows 16 rt + 0..15, one piece per lane) then fall
// on distinct banks, and its 8-byte writes (four columns of one row per
// lane) need two passes per sixteen lanes, the least any layout allows.
template <int D>
__device__ __forceinline__ int x_off(int row, int col) {
  return row * D + (((col >> 3) ^ (row & (D / 8 - 1))) << 3) + (col & 7);
}

// Operands of one frame held by one thread.
template <int D>
struct FrameRegs {
  f16x8 nk[ScanShape<D>::KS];                          // N column tile (k-slices of this lane)
  f16x8 b;                                             // row tile 0 in the low half, 1 in the high half (zero for
                                                       // d = 16): J_t / B' tiles in untransposed accumulator order,
                                                       // or B_t row segments
  float4 al;                                           // alpha of this lane's four columns
};

}  // namespace

template <int D, int MODE>
__global__ __launch_bounds__(ScanShape<D>::NT) void scan_kernel(ScanPair p) {
  static_assert(MODE == kFrameScan || MODE == kFrameScanB || MODE == kChunkScan || MODE == kSanaScan,
                "compose runs in compose_kernel");
  // frame slots of frame_kernel hold J_t in accumulator order, added after
  // the product; SANA-WM frame slots hold -A/U as the operand and B' in
  // accumulator order, added after the product together with X; the chunk
  // maps' J_c is added after the product in any case; only the Newton
  // comparator's slots hold B_t, added before the product
  constexpr bool POST = MODE != kFrameScanB;
  using SS = ScanShape<D>;
  constexpr int ROWS = SS::ROWS, NQ = SS::NQ, PD = SS::PD;
  static_assert(NQ == SS::RTS && NQ <= 2, "one half of FrameRegs::b per 16-row tile");
  // X = S Diag(alpha) as an f16 hi/lo pair, row-major, two buffers
  __shared__ __attribute__((aligned(16))) _Float16 sXh[2][ROWS * SS::XP];
  __shared__ __attribute__((aligned(16))) _Float16 sXl[2][ROWS * SS::XP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int RB = D / ROWS;  // row blocks per head
  // the row blocks of a head (and the heads of a direction) share an XCD
  int L = xcd_block(blockIdx.x, gridDim.x);
  const int per_dir = p.dir[0].H * RB;
  const int dir = L >= per_dir ? 1 : 0;
  L -= dir * per_dir;
  const ScanArgs& a = p.dir[dir];
  const int h = L / RB;
  const int r0 = ROWS * (L - h * RB);
  const int ct = wave;       // column tile of S this wavefront holds
  const int xc0 = 16 * ct + 4 * lg;  // this lane's four columns (of row r0 + 16 rt + lr)

  const size_t slot_floats = ws_slot_floats(D);
  const float* frames = a.frames + (size_t)h * a.n_eff * slot_floats;
  const float* alpha_h = a.alpha + (size_t)h * a.T * D;
  float* states_h = a.states + (size_t)h * a.count * D * D;
  // chunk maps of (head, direction, chunk c): 4 d^2 bytes
  auto chunk_map = [&](int c) {
    return static_cast<char*>(a.chunks) + ((size_t)(2 * h + a.reverse) * a.C + c) * (size_t)(4 * D * D);
  };
  // A frame's operands come in four parts, so that a step can issue the
  // loads of the frame PD steps ahead part by part between its own k-steps:
  // part 0: N's k-slices 0, 1; part 1: k-slices 2, 3; part 2: B; part 3: alpha.
  // What a frame slot holds after N (or the SANA-WM transition): J_t in
  // accumulator order at byte 2 d^2 (frame_kernel), B_t row-major at byte
  // 4 d^2 (the Newton comparator), or B' in accumulator order at byte 4 d^2
  // (SANA-WM).  The chunk scan reads frame slots only for the text step.
  const int form = MODE == kSanaScan ? 2 : (MODE == kFrameScanB || (MODE == kChunkScan && p.bform)) ? 1 : 0;
  auto load_part = [&](FrameRegs<D>& fr, int slot, const float* alpha_row, int part) {
    const float* base = frames + (size_t)slot * slot_floats;
    const _Float16* nf = reinterpret_cast<const _Float16*>(base);
    const _Float16* bm = reinterpret_cast<const _Float16*>(base + D * D);  // B_t, row-major
    const f16x4* ba = reinterpret_cast<const f16x4*>(form == 0 ? base + D * D / 2 : base + D * D);
    // fragment order: one wavefront reads 64 consecutive 16-byte chunks
#pragma unroll
    for (int kk = 0; kk < SS::KS; ++kk) {
      if (kk / 2 != part) continue;
      if (lg < SS::LG) {
        const int chunk = ((ct * SS::KS + kk) * SS::LG + lg) * 16 + lr;
        fr.nk[kk] = reinterpret_cast<const f16x8*>(nf)[chunk];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) fr.nk[kk][e] = (_Float16)0.f;
      }
    }
    if (part == 2) {
      f16x4 t[2] = {};
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        if (form == 1)
          t[q] = *reinterpret_cast<const f16x4*>(bm + (size_t)(r0 + 16 * q + lr) * D + xc0);
        else
          t[q] = ba[((r0 / 16 + q) * SS::NW + ct) * 64 + lane];
      }
      fr.b = __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7);
    }
    if (part == 3)
      fr.al = alpha_row ? *reinterpret_cast<const float4*>(alpha_row + xc0) : make_float4(1.f, 1.f, 1.f, 1.f);
  };
  auto load = [&](FrameRegs<D>& fr, int slot, const float* alpha_row) {
#pragma unroll
    for (int part = 0; part < 4; ++part) load_part(fr, slot, alpha_row, part);
  };

  // chunk scan: M_c as the B operand (fragment order, like N) and this
  // lane's accumulator-order J_c entries
  auto load_map_part = [&](FrameRegs<D>& fr, int c, int part) {
    const char* base = chunk_map(c);
    const _Float16* mf = reinterpret_cast<const _Float16*>(base);
    const f16x4* jf = reinterpret_cast<const f16x4*>(base + 2 * D * D);
#pragma unroll
    for (int kk = 0; kk < SS::KS; ++kk) {
      if (kk / 2 != part) continue;
      if (lg < SS::LG) {
        const int chunk = ((ct * SS::KS + kk) * SS::LG + lg) * 16 + lr;
        fr.nk[kk] = reinterpret_cast<const f16x8*>(mf)[chunk];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) fr.nk[kk][e] = (_Float16)0.f;
      }
    }
    if (part == 2) {
      f16x4 t[2] = {};
#pragma unroll
      for (int rt = 0; rt < SS::RTS; ++rt) t[rt] = jf[((r0 / 16 + rt) * SS::NW + ct) * 64 + lane];
      fr.b = __builtin_shufflevector(t[0], t[1], 0, 1, 2, 3, 4, 5, 6, 7);
    }
    if (part == 3) fr.al = make_float4(1.f, 1.f, 1.f, 1.f);
  };
  auto load_map = [&](FrameRegs<D>& fr, int c) {
#pragma unroll
    for (int part = 0; part < 4; ++part) load_map_part(fr, c, part);
  };

  // J_t, B' and J_c come in the untransposed accumulator order; transposed
  // against this identity they start the accumulators
  const f16x8 eye[2] = {eye_k32(lr, lg, 0), eye_k32(lr, lg, 1)};

  // The state: st[rt] holds S[r0 + 16 rt + lr][xc0 .. xc0 + 3].
  f32x4 st[SS::RTS];
  int xb = 0;  // LDS buffer of X for the next step

  // one frame write: S <- (S Diag(al) + B) N; a step with live == false
  // leaves S unchanged (padding at the end of the chain); with logits the
  // decay is sigmoid(al).  With post, B is added after the product,
  // S <- S Diag(al) N + B, B in untransposed accumulator order: one chunk
  // step S M_c + J_c (al = 1, fr from load_map), one frame step with J_t, or
  // one SANA-WM frame write.
  // next(part) issues part `part` of a later frame's loads; it is called
  // after each k-step's MFMAs, so that those loads leave this wavefront
  // while its MFMAs run instead of in one burst per step.
  auto step = [&](const FrameRegs<D>& fr, float* rec, bool live, bool logits, bool post, auto&& next) {
    float4 al = fr.al;
    if (logits) al = make_float4(sigmoid_gate(al.x), sigmoid_gate(al.y), sigmoid_gate(al.z), sigmoid_gate(al.w));
    _Float16* xh_buf = sXh[xb];
    _Float16* xl_buf = sXl[xb];
    f16x4 hi[SS::RTS], lo[SS::RTS];
#pragma unroll
    for (int rt = 0; rt < SS::RTS; ++rt) {
      float x[4] = {st[rt][0] * al.x, st[rt][1] * al.y, st[rt][2] * al.z, st[rt][3] * al.w};
      if (!post) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] += (float)fr.b[4 * rt + e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[rt][e] = (_Float16)x[e];
        lo[rt][e] = (_Float16)(x[e] - (float)hi[rt][e]);
      }
      *reinterpret_cast<f16x4*>(xh_buf + x_off<D>(16 * rt + lr, xc0)) = hi[rt];
      *reinterpret_cast<f16x4*>(xl_buf + x_off<D>(16 * rt + lr, xc0)) = lo[rt];
    }
    lds_barrier();
    f32x4 acc[SS::RTS];
#pragma unroll
    for (int rt = 0; rt < SS::RTS; ++rt) {
      if (post) {
        acc[rt] = transpose_tile(fr.b, eye[rt]);
        if constexpr (MODE == kSanaScan) {  // the identity part: X (I - A') = X + X (-A')
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[rt][e] += (float)hi[rt][e] + (float)lo[rt][e];
        }
      } else {
        acc[rt] = f32x4{0, 0, 0, 0};
      }
    }
    // every X fragment of the step is read before the first product, so
    // that the LDS latency is paid once per step, not once per k-step
    f16x8 xh[SS::KS][SS::RTS], xl[SS::KS][SS::RTS];
#pragma unroll
    for (int kk = 0; kk < SS::KS; ++kk) {
      const int k0 = 32 * kk + 8 * lg;
#pragma unroll
      for (int rt = 0; rt < SS::RTS; ++rt) {
        if (k0 < D) {
          xh[kk][rt] = *reinterpret_cast<const f16x8*>(xh_buf + x_off<D>(16 * rt + lr, k0));
          xl[kk][rt] = *reinterpret_cast<const f16x8*>(xl_buf + x_off<D>(16 * rt + lr, k0));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) xh[kk][rt][e] = xl[kk][rt][e] = (_Float16)0.f;
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of the products
#pragma unroll
    for (int kk = 0; kk < SS::KS; ++kk) {
#pragma unroll
      for (int rt = 0; rt < SS::RTS; ++rt) {
        acc[rt] = mfma_f16(fr.nk[kk], xh[kk][rt], acc[rt]);
        acc[rt] = mfma_f16(fr.nk[kk], xl[kk][rt], acc[rt]);
      }
      if (kk < 4) next(kk);
    }
#pragma unroll
    for (int part = SS::KS; part < 4; ++part) next(part);
    xb ^= 1;
#pragma unroll
    for (int rt = 0; rt < SS::RTS; ++rt) {
      if (live) st[rt] = acc[rt];
      if (rec) {
        bool fin = true;
#pragma unroll
        for (int e = 0; e < 4; ++e) fin = fin && __builtin_isfinite(acc[rt][e]);
        *reinterpret_cast<f32x4*>(rec + (size_t)(r0 + 16 * rt + lr) * D + xc0) = acc[rt];
        if (!fin) atomicOr(a.status, VDA_DEV_NONFINITE);
      }
    }
  };

  // ---- initial state
#pragma unroll
  for (int rt = 0; rt < SS::RTS; ++rt) {
    if (a.s_init)
      st[rt] = *reinterpret_cast<const f32x4*>(a.s_init + (size_t)h * D * D + (size_t)(r0 + 16 * rt + lr) * D + xc0);
    else
      st[rt] = f32x4{0, 0, 0, 0};
  }
  if (!a.s_init && a.use_text) {
    FrameRegs<D> fr;
    load(fr, a.n, nullptr);
    step(fr, nullptr, true, false, form != 1, [](int) {});  // S^T = 0 N_T + J_T (or (0 + B_T) N_T, or 0 T_T + B'_T)
  }
#pragma unroll
  for (int rt = 0; rt < SS::RTS; ++rt) {
    st[rt] *= a.scale;
    *reinterpret_cast<f32x4*>(states_h + (size_t)(r0 + 16 * rt + lr) * D + xc0) = st[rt];
  }

  if constexpr (MODE == kChunkScan) {
    // ---- C chunk steps S <- S M_c + J_c, maps prefetched PD chunks ahead;
    // the state is recorded after every chunk
    const int n = a.C;
    if (n == 0) return;
    auto slot_of = [&](int i) { return a.reverse ? n - 1 - i : i; };
    auto cl = [&](int i) { return i < n ? i : n - 1; };
    FrameRegs<D> fr[PD + 1];
#pragma unroll
    for (int j = 0; j < PD; ++j) load_map(fr[j], slot_of(cl(j)));
    for (int i0 = 0; i0 < n; i0 += PD + 1) {
#pragma unroll
      for (int j = 0; j <= PD; ++j) {
        const int i = i0 + j;
        // the maps' loads issued in one piece before the step (spreading them
        // over the k-steps, as the frame scan does, measured slower here)
        load_map(fr[(j + PD) % (PD + 1)], slot_of(cl(i + PD)));
        step(fr[j], i < n ? states_h + (size_t)(i + 1) * D * D : nullptr, i < n, false, true, [](int) {});
      }
    }
    return;
  }

  // ---- the chain, operands prefetched PD frames ahead (PD + 1 register sets).
  // Loads past the last frame re-read the last frame, so every step issues
  // the same loads and the wait before a step covers only that step's operands.
  const int n = a.n;
  if (n == 0) return;
  auto slot_of = [&](int i) { return a.reverse ? n - 1 - i : i; };
  auto alpha_of = [&](int i) { return alpha_h + (size_t)(a.a + slot_of(i)) * D; };
  auto cl = [&](int i) { return i < n ? i : n - 1; };
  auto rec_of = [&](int i) -> float* {
    const bool record = i < n && (((i + 1) % a.every == 0) || (i + 1 == n));
    return record ? states_h + (size_t)((i + a.every) / a.every) * D * D : nullptr;
  };
  // The chain runs in blocks of PD + 1 steps without an early exit (a single
  // loop exit keeps the waits before each step precise); steps past the last
  // frame are no-ops.
  FrameRegs<D> fr[PD + 1];
#pragma unroll
  for (int j = 0; j < PD; ++j) load(fr[j], slot_of(cl(j)), alpha_of(cl(j)));
  for (int i0 = 0; i0 < n; i0 += PD + 1) {
#pragma unroll
    for (int j = 0; j <= PD; ++j) {
      const int i = i0 + j;
      const int ns = slot_of(cl(i + PD));
      const float* na = alpha_of(cl(i + PD));
      step(fr[j], rec_of(i), i < n, a.prep != 0, POST,
           [&](int part) { load_part(fr[(j + PD) % (PD + 1)], ns, na, part); });
    }
  }
}

namespace {

template <int D>
struct ComposeShape {
  static constexpr int NTW = D == 128 ? 2 : 1;         // 16-row tiles of Z per wavefront
  static constexpr int NWH = D / (16 * NTW);            // wavefronts per d x d half of Z
  static constexpr int NTH = 2 * 64 * NWH;              // threads: both halves
  static constexpr int MT = D / 16;                     // 16-column tiles of Z
  static constexpr int KS = D >= 32 ? D / 32 : 1;       // MFMA k-steps (D = 16: one, zero padded)
  static constexpr int NCH = 2 * D * D / 16;            // 16-byte chunks of N
  static constexpr int CPT = (NCH + NTH - 1) / NTH;     // chunks staged per thread
  static constexpr int TP = D + 8;                      // LDS pitch (halves) of the output tiles
  static constexpr int NLDS = 2 * D * TP > 2 * D * D ? 2 * D * TP : 2 * D * D;  // halves
};

template <int D>
struct ComposeLds {
  _Float16 n[ComposeShape<D>::NLDS];  // N of two frames; then both output tiles
  float al[2][D];                     // alpha of two frames
};

}  // namespace

// The chunk maps of every (head, chunk, direction).  One workgroup runs one
// chain: its first half of wavefronts the d rows of Y (from I, no
// injection), its second half the d rows of X (from 0, with the injection);
// N and alpha of each frame are staged once for both.  A frame step is
// Z <- (Z Diag(alpha)) N + J_t on slots holding N_t and J_t, or
// Z <- (Z Diag(alpha) + B_t) N on slots holding N_t and B_t (BFORM, the
// Newton comparator).  The product is taken transposed, Z^T <- N X^T (N is
// symmetric), so that a lane's accumulators hold four consecutive columns of
// one row of Z: the next step's X is then formed in registers and is already
// the B operand of the next MFMAs, with the k order permuted so that k-slot
// group g covers columns 32kk + 4g .. +3 and 32kk + 16 + 4g .. +3 (both
// operands agree on it).  N's fragment order serves that order as two 8-byte
// LDS reads per operand.  N and alpha of the next frame are fetched during
// the current frame's MFMAs and staged into the other LDS buffer; one barrier
// per frame.  X enters the MFMA as an f16 hi/lo pair on the X rows (J_c keeps
// float32 accuracy) and as f16 on the Y rows (M_c: the product of
// contractions, whose rounding the f16 store of M_c dominates).
template <int D, bool BFORM>
__global__ __launch_bounds__(ComposeShape<D>::NTH, 1) void compose_kernel(ScanPair p) {
  using CS = ComposeShape<D>;
  constexpr int MT = CS::MT, NTW = CS::NTW, KS = CS::KS, TP = CS::TP;
  __shared__ __attribute__((aligned(16))) ComposeLds<D> lds;
  _Float16* sN = lds.n;
  float (*sA)[D] = lds.al;

  int L = xcd_block(blockIdx.x, gridDim.x);
  const int per_dir = p.dir[0].H * p.dir[0].C;
  const int dir = L >= per_dir ? 1 : 0;
  L -= dir * per_dir;
  const ScanArgs& a = p.dir[dir];
  const int h = L / a.C, cc = L - h * a.C;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const bool jpart = wave >= CS::NWH;                     // rows of J_c (else of M_c); wave-uniform
  const int n0 = 16 * NTW * (jpart ? wave - CS::NWH : wave);  // first row of Z (within its half)
  const int P = a.P;
  const size_t slot_floats = ws_slot_floats(D);
  const float* frames = a.frames + (size_t)h * a.n_eff * slot_floats;
  const float* alpha_h = a.alpha + (size_t)h * a.T * D;
  auto slot_of = [&](int i) { return P * cc + (a.reverse ? P - 1 - i : i); };

  f16x8 nreg[CS::CPT];
  float areg = 0.f;
  // per row tile nt, column tiles 2c and 2c + 1 in the two halves of
  // breg[nt][c] (the high half zero when MT is odd)
  constexpr int MP = (MT + 1) / 2;
  f16x8 breg[NTW][MP];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
    for (int c = 0; c < MP; ++c)
#pragma unroll
      for (int e = 0; e < 8; ++e) breg[nt][c][e] = (_Float16)0.f;
  const f16x8 eye[2] = {eye_k32(lr, lg, 0), eye_k32(lr, lg, 1)};
  auto put_b = [&](int nt, int mt, f16x4 v) {
#pragma unroll
    for (int e = 0; e < 4; ++e) breg[nt][mt / 2][4 * (mt & 1) + e] = v[e];
  };
  auto fetch = [&](int i) {
    const float* base = frames + (size_t)slot_of(i) * slot_floats;
    const f16x8* src = reinterpret_cast<const f16x8*>(base);
#pragma unroll
    for (int j = 0; j < CS::CPT; ++j) {
      const int c = tid + j * CS::NTH;
      if (c < CS::NCH) nreg[j] = src[c];
    }
    if (tid < D) areg = alpha_h[(size_t)(a.a + slot_of(i)) * D + tid];
    if (jpart && BFORM) {  // B_t[row][4 consecutive columns], row-major at byte 4 d^2
      const _Float16* bm = reinterpret_cast<const _Float16*>(base + D * D);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          put_b(nt, mt, *reinterpret_cast<const f16x4*>(bm + (size_t)(n0 + 16 * nt + lr) * D + 16 * mt + 4 * lg));
    } else if (jpart) {
      // J_t in the accumulator order at byte 2 d^2: this lane's f16x4 of
      // tile (R, mt), i.e. J[16R + 4 lg + e][16 mt + lr], loaded whole; it is
      // the transpose of what the accumulators need, which the product with
      // the identity at the start of each step provides (exactly)
      const f16x4* jm = reinterpret_cast<const f16x4*>(base + D * D / 2);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) put_b(nt, mt, jm[(size_t)(((n0 + 16 * nt) / 16) * MT + mt) * 64 + lane]);
    }
  };
  auto stage = [&](int buf) {
    f16x8* dst = reinterpret_cast<f16x8*>(sN + buf * D * D);
#pragma unroll
    for (int j = 0; j < CS::CPT; ++j) {
      const int c = tid + j * CS::NTH;
      if (c < CS::NCH) dst[c] = nreg[j];
    }
    if (tid < D) sA[buf][tid] = a.prep ? sigmoid_gate(areg) : areg;
  };

  // this half of Z in accumulators: acc[mt][nt][e] = Z[n0 + 16nt + lr][16mt + 4lg + e]
  f32x4 acc[MT][NTW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[mt][nt][e] = (!jpart && n0 + 16 * nt + lr == 16 * mt + 4 * lg + e) ? 1.f : 0.f;

  // the frames of the chunk on this half (JP: the X rows); both halves run
  // the same sequence of barriers
  auto run = [&](auto jp) {
    constexpr bool JP = decltype(jp)::value;
    fetch(0);
    stage(0);
    lds_barrier();
    for (int i = 0; i < P; ++i) {
      const int buf = i & 1;
      // X = Z Diag(alpha) (+ B) as the B operands of the k-steps
      f16x8 xh[NTW][KS], xl[NTW][KS];
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int mt = 2 * kk + half;
          if (mt < MT) {
            const float4 al = *reinterpret_cast<const float4*>(&sA[buf][16 * mt + 4 * lg]);
            const float alv[4] = {al.x, al.y, al.z, al.w};
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float x = (JP && BFORM) ? fmaf(acc[mt][nt][e], alv[e], (float)breg[nt][mt / 2][4 * (mt & 1) + e])
                                              : acc[mt][nt][e] * alv[e];
                const _Float16 hi = (_Float16)x;
                xh[nt][kk][4 * half + e] = hi;
                xl[nt][kk][4 * half + e] = JP ? (_Float16)(x - (float)hi) : (_Float16)0.f;
              }
          } else {
#pragma unroll
            for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
              for (int e = 0; e < 4; ++e) xh[nt][kk][4 * half + e] = xl[nt][kk][4 * half + e] = (_Float16)0.f;
          }
        }
      // Z^T <- N X^T (+ J_t^T, the accumulators' start: the loaded tile read
      // as an A operand is J_t^T's tile, and its product with the identity
      // lays it out as an accumulator)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          if constexpr (JP && !BFORM)
            acc[mt][nt] = transpose_tile(breg[nt][mt / 2], eye[mt & 1]);
          else
            acc[mt][nt] = f32x4{0, 0, 0, 0};
        }
      // the next frame's loads are in flight during the MFMAs
      if (i + 1 < P) fetch(i + 1);
      const _Float16* nb = sN + buf * D * D;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int m = 16 * mt + lr;
          const f16x4 lo4 = *reinterpret_cast<const f16x4*>(nb + ntile_chunk(D, m, 4 * kk + (lg >> 1)) * 8 + 4 * (lg & 1));
          f16x4 hi4;
          if (32 * kk + 16 < D) {
            hi4 = *reinterpret_cast<const f16x4*>(nb + ntile_chunk(D, m, 4 * kk + 2 + (lg >> 1)) * 8 + 4 * (lg & 1));
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) hi4[e] = (_Float16)0.f;
          }
          const f16x8 av = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) {
            acc[mt][nt] = mfma_f16(av, xh[nt][kk], acc[mt][nt]);
            if (JP) acc[mt][nt] = mfma_f16(av, xl[nt][kk], acc[mt][nt]);
          }
        }
      if (i + 1 < P) stage(buf ^ 1);
      lds_barrier();
    }
  };
  if (jpart)
    run(std::true_type{});
  else
    run(std::false_type{});

  // ---- store through LDS (the N buffers are free now): M_c from the first
  //      half of the tile memory, J_c from the second
  char* out = static_cast<char*>(a.chunks) + ((size_t)(2 * h + a.reverse) * a.C + cc) * (size_t)(4 * D * D);
  _Float16* TM = sN;
  _Float16* TJ = sN + D * TP;
  if (!jpart) {
    // T_M[m][n] = M_c[n][m]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e) TM[(16 * mt + 4 * lg + e) * TP + n0 + 16 * nt + lr] = (_Float16)acc[mt][nt][e];
  } else {
    // T_J[n][m] = J_c[n][m]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        f16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (_Float16)acc[mt][nt][e];
        *reinterpret_cast<f16x4*>(TJ + (n0 + 16 * nt + lr) * TP + 16 * mt + 4 * lg) = v;
      }
  }
  lds_barrier();
  // M_c as column chunks in the fragment order of N
  constexpr int LG = D >= 32 ? 4 : D / 8;
  f16x8* mf = reinterpret_cast<f16x8*>(out);
  for (int q = tid; q < D * D / 8; q += CS::NTH) {
    const int t = q / (16 * LG);
    const int c = 4 * (t % KS) + (q / 16) % LG;
    const int j = 16 * (t / KS) + (q & 15);
    mf[q] = *reinterpret_cast<const f16x8*>(TM + j * TP + 8 * c);
  }
  // J_c in the chunk scan's accumulator order
  f16x4* jf = reinterpret_cast<f16x4*>(out + 2 * D * D);
  for (int q = tid; q < D * D / 4; q += CS::NTH) {
    const int l = q & 63, t = q >> 6;
    const int rt = t / MT, ct = t - rt * MT;
    const int row = 16 * rt + 4 * (l >> 4), col = 16 * ct + (l & 15);
    f16x4 v;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = TJ[(row + e) * TP + col];
    jf[q] = v;
  }
}

int launch_scan(const ScanPair& p, int d, hipStream_t stream) {
  const int H = p.dir[0].H;
  if (H == 0) return 0;
  if (p.mode == kCompose) {
    if (p.dir[0].C == 0 || p.dir[0].P == 0) return 0;
    const long blocks = (long)p.ndir * H * p.dir[0].C;  // one workgroup per chain
#define VDA_COMPOSE(DD)                                                                               \
    if (d == DD) {                                                                                    \
      if (p.bform)                                                                                    \
        hipLaunchKernelGGL((compose_kernel<DD, true>), dim3((unsigned)blocks), dim3(ComposeShape<DD>::NTH), 0, stream, p); \
      else                                                                                            \
        hipLaunchKernelGGL((compose_kernel<DD, false>), dim3((unsigned)blocks), dim3(ComposeShape<DD>::NTH), 0, stream, p); \
      return 0;                                                                                       \
    }
    VDA_COMPOSE(16) VDA_COMPOSE(32) VDA_COMPOSE(64) VDA_COMPOSE(128)
#undef VDA_COMPOSE
    return -1;
  }
#define VDA_SCAN(DD, MM)                                                                             \
  if (d == DD && p.mode == MM) {                                                                     \
    const long blocks = (long)p.ndir * H * (DD / ScanShape<DD>::ROWS);                               \
    hipLaunchKernelGGL((scan_kernel<DD, MM>), dim3((unsigned)blocks), dim3(ScanShape<DD>::NT), 0, stream, p); \
    return 0;                                                                                        \
  }
#define VDA_SCAN_D(DD) \
  VDA_SCAN(DD, kFrameScan) VDA_SCAN(DD, kFrameScanB) VDA_SCAN(DD, kChunkScan) VDA_SCAN(DD, kSanaScan)
  VDA_SCAN_D(16) VDA_SCAN_D(32) VDA_SCAN_D(64) VDA_SCAN_D(128)
#undef VDA_SCAN_D
#undef VDA_SCAN
  return -1;
}

}  // namespace vda
