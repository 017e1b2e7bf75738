// Forward / reverse VDA scan: the only sequential part of the path.
//
//   S_t = (S_{t-1} Diag(alpha_t) + B_t) N_t,   N_t = (I + A_t)^{-1}
//
// ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream Video
// Generation", core-method section, paragraph 2: closed-form frame write;
// method-steps section, step (4): both scans start from the text state.)
//
// The d_v rows of S evolve independently (row i: s_t = (s_{t-1} * alpha_t +
// b_t) N_t), so one (head, direction) chain is split over d/16 workgroups of
// 16 rows each.  A workgroup keeps its 16 x d slice of S in LDS in float32.
// Per frame, the VALU forms X = S Diag(alpha) + B (float32) and splits it into
// bf16 hi/lo; each wavefront then computes 16 x (d/4) of X N on MFMA as
// X_hi N_hi + X_hi N_lo + X_lo N_hi (error about 2^-16 relative), with the N
// columns read as rows (N is symmetric).  The next frame's N, B rows and alpha
// are loaded into registers while the current frame is multiplied.
#include "vda_common.h"
#include "vda_kernels.h"

namespace vda {

namespace {

template <int D>
struct ScanShape {
  static constexpr int NW = (D / 16) < 4 ? (D / 16) : 4;  // active wavefronts
  static constexpr int CTW = (D / 16) / NW;               // 16-column tiles per wavefront
  static constexpr int KS = D / 32 > 0 ? D / 32 : 1;      // MFMA k-steps (D = 16: one, zero padded)
  static constexpr int EPT = 16 * D / kThreads;           // X elements per thread (>= 1)
  static constexpr int XP = D + 8;                        // LDS row pitch of X (halves)
};

// Registers holding one frame's operands for this thread.
template <int D>
struct FrameRegs {
  float n[ScanShape<D>::CTW][ScanShape<D>::KS][8];  // N columns of this wavefront's tiles
  float b[ScanShape<D>::EPT > 0 ? ScanShape<D>::EPT : 1];
  float al[ScanShape<D>::EPT > 0 ? ScanShape<D>::EPT : 1];
};

template <int D>
__device__ __forceinline__ void load_frame(FrameRegs<D>& fr, const float* slot, const float* alpha_row,
                                           int r0, int tid, int wave, int lane) {
  using S = ScanShape<D>;
  const int lr = lane & 15, lg = lane >> 4;
  if (wave < S::NW) {
#pragma unroll
    for (int i = 0; i < S::CTW; ++i) {
      const int col = 16 * (wave * S::CTW + i) + lr;
#pragma unroll
      for (int kk = 0; kk < S::KS; ++kk) {
        const int k0 = 32 * kk + 8 * lg;
#pragma unroll
        for (int e = 0; e < 8; ++e) fr.n[i][kk][e] = (k0 + e < D) ? slot[(size_t)col * D + k0 + e] : 0.f;
      }
    }
  }
  // X elements: row tid / (D / EPT), columns contiguous
  constexpr int TPR = D / S::EPT;  // threads per row
  const int row = tid / TPR, c0 = (tid - row * TPR) * S::EPT;
  if (row < 16) {
#pragma unroll
    for (int e = 0; e < S::EPT; ++e) {
      fr.b[e] = slot[(size_t)D * D + (size_t)(r0 + row) * D + c0 + e];
      fr.al[e] = alpha_row ? alpha_row[c0 + e] : 1.f;
    }
  }
}

}  // namespace

template <int D>
__global__ __launch_bounds__(kThreads) void scan_kernel(ScanArgs a) {
  using S = ScanShape<D>;
  __shared__ __attribute__((aligned(16))) float sS[16 * D];
  __shared__ __attribute__((aligned(16))) __bf16 sXh[16 * S::XP];
  __shared__ __attribute__((aligned(16))) __bf16 sXl[16 * S::XP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  constexpr int RB = D / 16;
  const int h = blockIdx.x / RB;
  const int r0 = 16 * (blockIdx.x - h * RB);
  constexpr int TPR = D / S::EPT;
  const int xrow = tid / TPR, xc0 = (tid - xrow * TPR) * S::EPT;

  const float* frames = a.frames + (size_t)h * a.n_eff * ws_slot_floats(D);
  const float* alpha_h = a.alpha + (size_t)h * a.T * D;
  float* states_h = a.states + (size_t)h * a.count * D * D;

  // one frame write on the LDS state slice: S <- (S Diag(al) + B) N
  auto step = [&](const FrameRegs<D>& fr, float* rec) {
    if (xrow < 16) {
#pragma unroll
      for (int e = 0; e < S::EPT; ++e) {
        const float x = fmaf(sS[xrow * D + xc0 + e], fr.al[e], fr.b[e]);
        __bf16 hi, lo;
        split_bf16(x, hi, lo);
        sXh[xrow * S::XP + xc0 + e] = hi;
        sXl[xrow * S::XP + xc0 + e] = lo;
      }
    }
    __syncthreads();
    if (wave < S::NW) {
#pragma unroll
      for (int i = 0; i < S::CTW; ++i) {
        const int ct = wave * S::CTW + i;
        f32x4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < S::KS; ++kk) {
          const int k0 = 32 * kk + 8 * lg;
          bf16x8 xh, xl, nh, nl;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const bool in = k0 + e < D;
            xh[e] = in ? sXh[lr * S::XP + k0 + e] : bits_to_bf16(0);
            xl[e] = in ? sXl[lr * S::XP + k0 + e] : bits_to_bf16(0);
            __bf16 hi, lo;
            split_bf16(fr.n[i][kk][e], hi, lo);
            nh[e] = hi;
            nl[e] = lo;
          }
          acc = mfma_bf16(xh, nh, acc);
          acc = mfma_bf16(xh, nl, acc);
          acc = mfma_bf16(xl, nh, acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sS[(4 * lg + e) * D + 16 * ct + lr] = acc[e];
          if (rec) rec[(size_t)(r0 + 4 * lg + e) * D + 16 * ct + lr] = acc[e];
        }
      }
    }
    __syncthreads();
  };

  // ---- initial state
  for (int i = tid; i < 16 * D; i += kThreads) sS[i] = 0.f;
  __syncthreads();
  if (a.s_init) {
    const float* si = a.s_init + (size_t)h * D * D;
    for (int i = tid; i < 16 * D; i += kThreads) sS[i] = si[(size_t)r0 * D + i];
    __syncthreads();
  } else if (a.use_text) {
    FrameRegs<D> fr;
    load_frame<D>(fr, frames + (size_t)a.n * ws_slot_floats(D), nullptr, r0, tid, wave, lane);
    step(fr, nullptr);  // S^T = (0 + B_T) N_T
  }
  for (int i = tid; i < 16 * D; i += kThreads) {
    const float s0 = a.scale * sS[i];
    sS[i] = s0;
    states_h[(size_t)r0 * D + i] = s0;
  }
  __syncthreads();

  // ---- the chain, with the next frame's operands prefetched
  if (a.n == 0) return;
  FrameRegs<D> cur, nxt;
  {
    const int f0 = a.reverse ? a.n - 1 : 0;
    load_frame<D>(cur, frames + (size_t)f0 * ws_slot_floats(D), alpha_h + (size_t)(a.a + f0) * D, r0, tid,
                  wave, lane);
  }
  for (int i = 0; i < a.n; ++i) {
    if (i + 1 < a.n) {
      const int f1 = a.reverse ? a.n - 2 - i : i + 1;
      load_frame<D>(nxt, frames + (size_t)f1 * ws_slot_floats(D), alpha_h + (size_t)(a.a + f1) * D, r0, tid,
                    wave, lane);
    }
    const bool record = ((i + 1) % a.every == 0) || (i + 1 == a.n);
    const int j = (i + a.every) / a.every;  // index of the state after i + 1 frames
    step(cur, record ? states_h + (size_t)j * D * D : nullptr);
    cur = nxt;
  }
}

int launch_scan(const ScanArgs& a, int d, hipStream_t stream) {
  if (a.H == 0) return 0;
  dim3 block(kThreads);
#define VDA_SCAN(DD)                                                                   \
  if (d == DD) {                                                                       \
    hipLaunchKernelGGL((scan_kernel<DD>), dim3((unsigned)(a.H * (DD / 16))), block, 0, \
                       stream, a);                                                     \
    return 0;                                                                          \
  }
  VDA_SCAN(16) VDA_SCAN(32) VDA_SCAN(64) VDA_SCAN(128)
#undef VDA_SCAN
  return -1;
}

}  // namespace vda
