// Forward / reverse VDA scan: the only sequential part of the path.
//
//   S_t = (S_{t-1} Diag(alpha_t) + B_t) N_t,   N_t = (I + A_t)^{-1}
//
// ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
// Generation", core-method section, paragraph 2: closed-form frame write;
// method-steps section, step (4): both scans start from the text state.)
//
// The d_v rows of S evolve independently (row i: s_t = (s_{t-1} * alpha_t +
// b_t) N_t), so one (head, direction) chain is split over d/32 workgroups of
// 32 rows each (16 for d = 16); the row blocks of a head are mapped to one
// XCD so that they share that XCD's L2 copy of N_t.  A workgroup keeps its
// 32 x d slice of S in LDS in float32 and runs d/16 wavefronts, one per
// 16-column output tile.
// Per frame, the VALU forms X = S Diag(alpha) + B (float32) and splits it into
// an f16 hi/lo pair in LDS; each wavefront computes its 16 x 16 tile of X N
// on MFMA as X_hi N + X_lo N, N being stored by the prepare kernel as f16 in
// MFMA fragment order and read as rows (N is symmetric).  Each workgroup
// pulls N and its rows of B through its CU's vector-memory path once per
// frame, and that is what bounds a step, so N and B are kept to 2 bytes per
// entry (f16).
// The chain is bound by the latency of these per-frame operand loads, so
// frames are prefetched three or four steps ahead into registers; the barriers wait
// for LDS traffic only, so the global loads stay in flight across them.
#include "vda_common.h"
#include "vda_kernels.h"

namespace vda {

namespace {

template <int D>
struct ScanShape {
  static constexpr int ROWS = D < 32 ? D : 32;          // state rows per workgroup
  static constexpr int RTS = ROWS / 16;                 // 16-row tiles per workgroup
  static constexpr int NW = D / 16;                     // wavefronts = 16-column tiles
  static constexpr int NT = 64 * NW;                    // threads
  static constexpr int KS = D >= 32 ? D / 32 : 1;       // MFMA k-steps (D = 16: one, zero padded)
  static constexpr int XP = D + 8;                      // LDS row pitch of X (halves)
  static constexpr int NQ = ROWS / 16;                  // float4 X chunks per thread
  static constexpr int TPR = D / 4;                     // threads per row in the elementwise phase
  static constexpr int LG = D >= 32 ? 4 : D / 8;        // k-chunk groups per fragment-order block
  static constexpr int PD = D >= 128 ? 3 : (D >= 64 ? 4 : 2);  // frames prefetched ahead
};

// Operands of one frame held by one thread.
template <int D>
struct FrameRegs {
  f16x8 nk[ScanShape<D>::KS];                          // N column tile (k-slices of this lane)
  f16x4 b[ScanShape<D>::NQ];                           // B row segments (rows xrow + 16 q)
  float4 al;                                           // alpha segment
};

}  // namespace

template <int D>
__global__ __launch_bounds__(ScanShape<D>::NT) void scan_kernel(ScanPair p) {
  using SS = ScanShape<D>;
  constexpr int ROWS = SS::ROWS, NQ = SS::NQ, PD = SS::PD;
  __shared__ __attribute__((aligned(16))) float sS[ROWS * D];
  __shared__ __attribute__((aligned(16))) _Float16 sXh[ROWS * SS::XP];
  __shared__ __attribute__((aligned(16))) _Float16 sXl[ROWS * SS::XP];

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
  // elementwise phase: thread owns columns xc0..xc0+3 of rows xrow + 16 q
  const int xrow = tid / SS::TPR, xc0 = 4 * (tid - xrow * SS::TPR);
  const int ct = wave;  // output column tile

  const size_t slot_floats = ws_slot_floats(D);
  const float* frames = a.frames + (size_t)h * a.n_eff * slot_floats;
  const float* alpha_h = a.alpha + (size_t)h * a.T * D;
  float* states_h = a.states + (size_t)h * a.count * D * D;

  auto load = [&](FrameRegs<D>& fr, int slot, const float* alpha_row) {
    const float* base = frames + (size_t)slot * slot_floats;
    const _Float16* nf = reinterpret_cast<const _Float16*>(base);
    const _Float16* bm = reinterpret_cast<const _Float16*>(base + D * D);
    // fragment order: one wavefront reads 64 consecutive 16-byte chunks
#pragma unroll
    for (int kk = 0; kk < SS::KS; ++kk) {
      if (lg < SS::LG) {
        const int chunk = ((ct * SS::KS + kk) * SS::LG + lg) * 16 + lr;
        fr.nk[kk] = reinterpret_cast<const f16x8*>(nf)[chunk];
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) fr.nk[kk][e] = (_Float16)0.f;
      }
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q)
      fr.b[q] = *reinterpret_cast<const f16x4*>(bm + (size_t)(r0 + xrow + 16 * q) * D + xc0);
    fr.al = alpha_row ? *reinterpret_cast<const float4*>(alpha_row + xc0) : make_float4(1.f, 1.f, 1.f, 1.f);
  };

  // one frame write on the LDS state slice: S <- (S Diag(al) + B) N; a step
  // with live == false leaves S unchanged (padding at the end of the chain);
  // with logits the decay is sigmoid(al)
  auto step = [&](const FrameRegs<D>& fr, float* rec, bool live, bool logits) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int row = xrow + 16 * q;
      const float4 s = *reinterpret_cast<const float4*>(sS + row * D + xc0);
      float4 al = fr.al;
      if (logits) al = make_float4(sigmoid_gate(al.x), sigmoid_gate(al.y), sigmoid_gate(al.z), sigmoid_gate(al.w));
      const f16x4 bb = fr.b[q];
      const float x[4] = {fmaf(s.x, al.x, (float)bb[0]), fmaf(s.y, al.y, (float)bb[1]),
                          fmaf(s.z, al.z, (float)bb[2]), fmaf(s.w, al.w, (float)bb[3])};
      f16x4 hi, lo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hi[e] = (_Float16)x[e];
        lo[e] = (_Float16)(x[e] - (float)hi[e]);
      }
      *reinterpret_cast<f16x4*>(sXh + row * SS::XP + xc0) = hi;
      *reinterpret_cast<f16x4*>(sXl + row * SS::XP + xc0) = lo;
    }
    lds_barrier();
    f32x4 acc[SS::RTS];
#pragma unroll
    for (int rt = 0; rt < SS::RTS; ++rt) acc[rt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < SS::KS; ++kk) {
      const int k0 = 32 * kk + 8 * lg;
#pragma unroll
      for (int rt = 0; rt < SS::RTS; ++rt) {
        f16x8 xh, xl;
        if (k0 < D) {
          xh = *reinterpret_cast<const f16x8*>(sXh + (16 * rt + lr) * SS::XP + k0);
          xl = *reinterpret_cast<const f16x8*>(sXl + (16 * rt + lr) * SS::XP + k0);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) xh[e] = xl[e] = (_Float16)0.f;
        }
        acc[rt] = mfma_f16(xh, fr.nk[kk], acc[rt]);
        acc[rt] = mfma_f16(xl, fr.nk[kk], acc[rt]);
      }
    }
#pragma unroll
    for (int rt = 0; rt < SS::RTS; ++rt) {
      if (live) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sS[(16 * rt + 4 * lg + e) * D + 16 * ct + lr] = acc[rt][e];
      }
      if (rec) {
#pragma unroll
        for (int e = 0; e < 4; ++e) rec[(size_t)(r0 + 16 * rt + 4 * lg + e) * D + 16 * ct + lr] = acc[rt][e];
      }
    }
    lds_barrier();
  };

  // ---- initial state
  if (a.s_init) {
    const float* si = a.s_init + (size_t)h * D * D + (size_t)r0 * D;
    for (int i = tid; i < ROWS * D; i += SS::NT) sS[i] = si[i];
  } else {
    for (int i = tid; i < ROWS * D; i += SS::NT) sS[i] = 0.f;
  }
  lds_barrier();
  if (!a.s_init && a.use_text) {
    FrameRegs<D> fr;
    load(fr, a.n, nullptr);
    step(fr, nullptr, true, false);  // S^T = (0 + B_T) N_T
  }
  for (int i = tid; i < ROWS * D; i += SS::NT) {
    const float s0 = a.scale * sS[i];
    sS[i] = s0;
    states_h[(size_t)r0 * D + i] = s0;
  }
  lds_barrier();

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
      load(fr[(j + PD) % (PD + 1)], slot_of(cl(i + PD)), alpha_of(cl(i + PD)));
      step(fr[j], rec_of(i), i < n, a.prep != 0);
    }
  }
}

int launch_scan(const ScanPair& p, int d, hipStream_t stream) {
  const int H = p.dir[0].H;
  if (H == 0) return 0;
#define VDA_SCAN(DD)                                                                              \
  if (d == DD) {                                                                                  \
    hipLaunchKernelGGL((scan_kernel<DD>), dim3((unsigned)(p.ndir * H * (DD / ScanShape<DD>::ROWS))), \
                       dim3(ScanShape<DD>::NT), 0, stream, p);                                    \
    return 0;                                                                                     \
  }
  VDA_SCAN(16) VDA_SCAN(32) VDA_SCAN(64) VDA_SCAN(128)
#undef VDA_SCAN
  return -1;
}

}  // namespace vda
