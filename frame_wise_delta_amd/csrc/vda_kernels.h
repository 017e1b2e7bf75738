// Kernel argument blocks and launchers (internal to libvda).
#pragma once

#include "vda_common.h"

namespace vda {

struct PrepArgs {
  const void* k;
  const void* v;
  const float* beta;
  const void* kt;
  const void* vt;
  const float* bt;
  float* frames;  // workspace after the header: [H][n_eff][N | B]
  int* status;
  int H, T, U, a, n, n_eff, Nt;
  int s0, cnt;    // frame slots [s0, s0 + cnt) of every head (slot n = text)
  int prep;       // k, k_text raw (L2-normalised here), beta, beta_text logits
};

struct ScanArgs {
  const float* frames;  // workspace frames: [H][n_eff][N | B]
  const float* alpha;   // [H][T][d]
  const float* s_init;  // [H][d][d] or nullptr
  float* states;        // [H][count][d][d]
  int H, T, a, n, n_eff, count;
  int every;            // record the state after every `every` frames
  int reverse;
  int use_text;         // S_init = S^T from the text slot (slot n) when s_init == nullptr
  float scale;
  int prep;             // alpha holds logits (the gate is sigmoid(logit))
  int* status;          // device status word (a non-finite recorded state sets VDA_DEV_NONFINITE)
  // chunk maps (compose and chunk-scan launches): per head, direction and
  // chunk, 4 d^2 bytes: M_c (f16, the fragment order of N) then J_c (f16,
  // accumulator order, see vda_scan.hip)
  void* chunks;
  int C, P;
};

// What a scan launch runs.
enum ScanMode {
  kFrameScan = 0,   // S_t = (S_{t-1} Diag(alpha_t)) N_t + J_t over the frames (slots from frame_kernel)
  kCompose = 1,     // the chunk maps (M_c, J_c) of every chunk, in parallel
  kChunkScan = 2,   // S_c = S_{c-1} M_c + J_c over the chunks
  kSanaScan = 3,    // S_t = X + X (-A_t/U) + B'_t, X = S_{t-1} Diag(alpha_t) (the SANA-WM comparator)
  kFrameScanB = 4,  // S_t = (S_{t-1} Diag(alpha_t) + B_t) N_t (slots holding N_t and B_t: the Newton comparator)
};

// One or two scans in one launch: blocks [0, H RB) run dir[0], the next
// H RB blocks (when ndir == 2) run dir[1] (compose: H C 2RB blocks per
// direction).
struct ScanPair {
  ScanArgs dir[2];
  int ndir;
  int mode;    // ScanMode
  int bform;   // compose: the slots hold N_t and B_t (else N_t and J_t)
};

struct ReadArgs {
  const void* q;          // [H][T][U][d]
  const float* alpha;     // [H][T][d]
  const float* sf;        // [H][count][d][d]
  const float* sr;        // [H][count][d][d] or nullptr (full mode)
  void* out;              // [H][T][U][d]
  int H, T, U, a, n, P, C, w, count;
  int bridge;
  int prep;               // q raw (L2-normalised here), alpha logits
  // readout epilogue (gated launches only): y = rmsnorm(o) * normw * sigmoid(gate)
  const void* gate;       // [H][T][U][d] logits, input dtype
  const float* normw;     // [H][d]
  float eps;
};

struct AttnArgs {
  const void* q;          // [H][T][U][d] bf16 (after the branch's QK normalisation and rotary encoding)
  const void* k;          // [H][T][U][d] bf16
  const void* v;          // [H][T][U][d] bf16 or f16 (v_f16)
  const void* kt;         // [H][Nt][d] bf16 or nullptr (Nt = 0)
  const void* vt;         // [H][Nt][d] like v, or nullptr
  void* out;              // [H][T][U][d]
  int H, T, U, a, P, C, w, Nt;
  float scale;
  int v_f16;              // v, vt are f16 (else bf16)
  int tiles_per_head, anchor_tiles, chunk_tiles;  // 256-query workgroups
};

// Statistics, factorisation and injection in one kernel: N_t and J_t = B_t N_t.
int launch_frame(const PrepArgs& a, int d, bool in_f32, hipStream_t stream);
// Statistics alone (the comparators): the upper tiles of A_t (float32) and B_t (f16).
int launch_stats(const PrepArgs& a, int d, bool in_f32, hipStream_t stream);
// N = (I + A)^{-1} by Newton iteration instead of Gauss-Jordan.
int launch_ns(const PrepArgs& a, int d, hipStream_t stream);
// SANA-WM comparator: -A/U and B' = B/sqrt(U) in place of N and B.
int launch_sana(const PrepArgs& a, int d, hipStream_t stream);
void launch_clear_status(int* status, hipStream_t stream);
// *dst = *src on the device (the status word of a workspace to a caller's int).
void launch_copy_status(const int* src, int32_t* dst, hipStream_t stream);
int launch_scan(const ScanPair& p, int d, hipStream_t stream);
int launch_readout(const ReadArgs& a, int d, int in_dtype, int out_dtype, hipStream_t stream);
// The readout with the RMSNorm + sigmoid-gate epilogue (a.gate, a.normw, a.eps).
int launch_readout_gated(const ReadArgs& a, int d, int in_dtype, int out_dtype, hipStream_t stream);
int launch_attn(const AttnArgs& a, int d, int out_dtype, hipStream_t stream);
// The index maps computed on the device by chunk_window / frame_chunk_of,
// the functions the readout and attention kernels use.
void launch_index_map(int C, int T, int w, int P, int a, int n, int32_t* rows, int32_t* frame_chunk,
                      hipStream_t stream);

}  // namespace vda
