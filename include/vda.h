/*
 * libvda — Video Delta Attention (VDA) linear branch on AMD MI355X (gfx950).
 *
 * The operation is defined on the summary page of the paper "Video DeltaNet:
 * A Video-Native Hybrid Attention for Livestream Video Generation"
 * (paper.rainbus.top, paper 2609.20744), cited as [VDN <section>]:
 *
 *   frame statistics   A_t = K_t^T Diag(beta_t) K_t,  B_t = V_t^T Diag(beta_t) K_t
 *                      [VDN 方法步骤详情 step (3)]
 *   frame write        S_t = (S_{t-1} Diag(alpha_t) + B_t)(I + A_t)^{-1}
 *                      [VDN 核心方法 para 2; 前置知识 "Delta 规则"]
 *   bidirectional scan forward and reverse over the non-anchor frames, both
 *                      started from text_init_scale * S^T
 *                      [VDN 核心方法 para 1; 方法步骤详情 step (4)]
 *   readout            o = S^f_{F(c)} (b_f * q) + S^r_{R(c)} (b_r * q), which
 *                      excludes the chunk-aligned softmax window and carries
 *                      each state to the query frame through the decay bridge
 *                      prod alpha_r [VDN 核心方法 para 1; 方法步骤详情 step (5)]
 *
 * Notation: H heads, T frames (anchors included), U tokens per frame,
 * d = d_k = d_v, P frames per chunk, n = T - 2*anchors scanned frames,
 * C = ceil(n / P) chunks.  The state S is d_v x d_k (row = value channel,
 * column = key channel) and is read as S q.
 *
 * Conventions (all entry points):
 *  - Layouts are dense row-major: q/k/v/out [H][T][U][d], beta [H][T][U]
 *    float32, alpha [H][T][d] float32, k_text/v_text [H][N_text][d],
 *    beta_text [H][N_text] float32, states [H][count][d][d] float32.
 *  - Every array pointer is a device pointer (hipMalloc'd or equivalent),
 *    16-byte aligned.  The caller owns every buffer; the library allocates no
 *    device memory and keeps no pointer after a call returns.
 *  - Calls that take `stream` only enqueue work on that hipStream_t (NULL =
 *    the null stream) and return without synchronising.  Buffers must stay
 *    alive until the caller synchronises the stream.
 *  - Every argument is validated on the host before anything is enqueued; a
 *    failed validation returns a negative code, launches nothing and leaves
 *    the message in vda_last_error() (thread-local).  No exception or abort
 *    crosses the ABI.
 *  - Numerical faults found on the device (a non-finite statistic or a
 *    non-positive pivot in the factorisation) set bits in a status word in
 *    the workspace; vda_device_status() reads it.
 */
#ifndef VDA_H
#define VDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
enum {
  VDA_OK = 0,
  VDA_ERR_NULL = -1,      /* a required pointer is NULL */
  VDA_ERR_SHAPE = -2,     /* inconsistent or unsupported sizes */
  VDA_ERR_DTYPE = -3,     /* unsupported element type */
  VDA_ERR_ALIGN = -4,     /* a pointer is not 16-byte aligned */
  VDA_ERR_WORKSPACE = -5, /* workspace too small */
  VDA_ERR_HIP = -6,       /* a HIP runtime call or kernel launch failed */
  VDA_ERR_DEVICE = -7,    /* no usable gfx950 device */
  VDA_ERR_VALUE = -8      /* a scalar argument is out of range */
};

/* element types */
enum { VDA_F32 = 0, VDA_BF16 = 1, VDA_F16 = 2 };

/* vda_desc.flags */
enum {
  VDA_NO_BRIDGE = 1u << 0, /* readout without the decay bridge (b_f = b_r = 1) */
  VDA_PREP = 1u << 1,      /* inputs are raw projections, prepared inside the kernels
                              [VDN 方法步骤详情 step (2)]: q, k and k_text are
                              L2-normalised per token, x / sqrt(||x||^2 + 1e-6), and
                              beta, beta_text and alpha are logits whose gates are
                              sigmoid(logit) */
  VDA_CHUNK_SCAN = 1u << 2, /* the scans run at chunk level [VDN 方法步骤详情 step (4)]:
                              vda_compose_chunks turns each chunk's P frame writes
                              into one affine map (M_c, J_c) and the scans apply
                              S <- S M_c + J_c once per chunk; needs window >= 0
                              and a larger workspace (vda_workspace_bytes) */
  VDA_SANA_WM = 1u << 3    /* comparator: the SANA-WM batched additive update
                              [VDN 核心方法 para 2] in place of the VDA write,
                              S_t = S_{t-1} Diag(alpha_t) (I - A_t/U) + B_t/sqrt(U)
                              (keys scaled by 1/sqrt(U), U the tokens of the frame;
                              N_text for the text write, so S^T = B_T/sqrt(N_text));
                              vda_prepare_frames then stores -A_t/U and
                              B_t/sqrt(U) in place of N_t and J_t; not with
                              VDA_CHUNK_SCAN */,
  VDA_NEWTON = 1u << 4     /* (I + A_t)^{-1} by Newton iteration
                              [VDN 实验结果, weaknesses: Newton iteration in place
                              of the exact inverse] instead of Gauss-Jordan:
                              X <- X + (I - G X) X from X_0 = 2/(1+g) I, g the largest
                              absolute row sum of G = I + A_t, until the residual
                              bound ((g-1)/(g+1))^(2^k) <= 1e-6; same workspace
                              contents and layout; not with VDA_SANA_WM */
};

/* bits of the device status word */
enum {
  VDA_DEV_NONFINITE = 1, /* a frame statistic, factor or recorded state was NaN/Inf */
  VDA_DEV_PIVOT = 2      /* I + A_t had a pivot <= 0 (not positive definite) */
};

typedef struct vda_desc {
  int32_t heads;       /* H >= 0 */
  int32_t frames;      /* T >= 2*anchors */
  int32_t tokens;      /* U >= 0 tokens per frame */
  int32_t d_k, d_v;    /* d_k == d_v, one of 16, 32, 64, 128 */
  int32_t chunk;       /* P >= 1 frames per chunk (5 for the VAE chunks) */
  int32_t anchors;     /* 1: frames 0 and T-1 are anchors; 0: none */
  int32_t window;      /* w >= 0: the softmax window of query chunk c is chunks
                          c-w..c+w clipped to [0, C-1] and n % P must be 0;
                          -1: no exclusion, the readout of frame t is S^f_t q
                          with S^f_t the forward state after frame t */
  int32_t text_tokens; /* N_text >= 0 text tokens forming S^T (0: S^T = 0) */
  int32_t in_dtype;    /* q, k, v, k_text, v_text: VDA_F32 or VDA_BF16 */
  int32_t out_dtype;   /* out: VDA_F32, VDA_BF16 or VDA_F16 */
  float text_init_scale; /* both scans start from text_init_scale * S^T;
                            1/2 reads the page's "initialised by halves" */
  uint32_t flags;      /* VDA_NO_BRIDGE | VDA_PREP | VDA_CHUNK_SCAN | VDA_SANA_WM | VDA_NEWTON */
} vda_desc;

/* Bytes of device workspace vda_prepare_frames needs for `desc` (host only,
 * enqueues nothing).  The workspace carries, per head, N_t = (I + A_t)^{-1}
 * and J_t = B_t N_t of every scanned frame and of the text "frame" (8 d^2
 * bytes per slot), plus the device status word, from vda_prepare_frames to
 * the scans.  With
 * VDA_CHUNK_SCAN it also holds the chunk maps of both directions
 * (4 d^2 bytes per head, direction and chunk). */
int vda_workspace_bytes(const vda_desc* desc, size_t* bytes);

/* Number of states each scan records per head (host only):
 * C + 1 when window >= 0 (the state after 0, 1, ..., C chunks),
 * n + 1 when window == -1 (the state after 0, 1, ..., n frames). */
int vda_state_count(const vda_desc* desc, int32_t* count);

/* Integer index maps (host only, host pointers) [VDN 核心方法 para 1]:
 *  chunk_rows [C][7] int32: (c, lo, hi, ws, we, F, R) — window chunks lo..hi
 *    = c-w..c+w clipped (w = 0 when window == -1), first/last window frame
 *    ws/we, F = lo (forward state index: chunks wholly before the window),
 *    R = C-1-hi (reverse state index: chunks wholly after the window);
 *  frame_chunk [T] int32: chunk of each frame, -1 for anchors.
 * Either pointer may be NULL to skip that output. */
int vda_index_map(const vda_desc* desc, int32_t* chunk_rows, int32_t* frame_chunk);

/* The same maps computed on the device, by the device code the readout and
 * the softmax branch take their windows from (a check that the two copies
 * of the map arithmetic agree).  chunk_rows [C][7] and frame_chunk [T] are
 * 16-byte aligned device pointers (each may be NULL only when its size is
 * 0); enqueues one small kernel on `stream`. */
int vda_index_map_device(const vda_desc* desc, int32_t* chunk_rows, int32_t* frame_chunk, void* stream);

/* Frame statistics and factorisation [VDN 方法步骤详情 step (3)]: for every
 * head and every scanned frame t (and the text tokens when text_tokens > 0)
 * computes A_t = K_t^T Diag(beta_t) K_t and B_t = V_t^T Diag(beta_t) K_t
 * over the frame's U tokens, factorises I + A_t and stores, per slot,
 *   N_t = (I + A_t)^{-1}  and  J_t = B_t N_t
 * in `ws` (f16 each), so that the frame write is
 * S_t = (S_{t-1} Diag(alpha_t)) N_t + J_t [VDN 核心方法 para 2].  Also
 * clears the device status word.  With VDA_NEWTON the slots hold N_t (by
 * Newton iteration) and B_t instead, and the scans form
 * (S_{t-1} Diag(alpha_t) + B_t) N_t; with VDA_SANA_WM they hold the
 * comparator's -A_t/U and B_t/sqrt(U).
 *  k, v        [H][T][U][d] in_dtype (anchor frames are not read)
 *  beta        [H][T][U] float32
 *  k_text, v_text [H][N_text][d] in_dtype; beta_text [H][N_text] float32
 *              (all three may be NULL when text_tokens == 0)
 *  ws          device workspace of ws_bytes >= vda_workspace_bytes(desc),
 *              256-byte aligned.
 * Value range: the kernels take K, beta*K and beta*V as f16 operands and
 * keep N_t, J_t (and B_t) as f16, so every |beta_u v_u|, every entry of
 * B_t (a sum over the frame's tokens of beta_u v_u k_u^T) and of J_t, and
 * every state entry must stay below 65504 in magnitude; a value that does
 * not becomes non-finite and sets VDA_DEV_NONFINITE.  L2-normalised keys and
 * values of unit scale are far inside this range. */
int vda_prepare_frames(const vda_desc* desc, const void* k, const void* v, const float* beta,
                       const void* k_text, const void* v_text, const float* beta_text,
                       void* ws, size_t ws_bytes, void* stream);

/* Chunk composition [VDN 方法步骤详情 step (4): chunk-level scan
 * S_out = S_in M_chunk + J_chunk], for descriptors with VDA_CHUNK_SCAN: with
 * M_t = Diag(alpha_t) N_t and J_t = B_t N_t (so that the frame write is
 * S_t = S_{t-1} M_t + J_t), stores for every head and chunk c the forward map
 * (M_c, J_c) = the composition of the chunk's frame maps in increasing frame
 * order, and the reverse map, composed in decreasing order.  M_c and J_c are
 * kept as f16 in `ws`; every chunk is composed independently.
 *  ws     holds the output of vda_prepare_frames for the same desc;
 *         ws_bytes >= vda_workspace_bytes(desc)
 *  alpha  [H][T][d] float32 (logits with VDA_PREP)
 * Returns VDA_ERR_SHAPE when desc lacks VDA_CHUNK_SCAN. */
int vda_compose_chunks(const vda_desc* desc, void* ws, size_t ws_bytes, const float* alpha, void* stream);

/* Forward scan [VDN 核心方法 para 1; 方法步骤详情 step (4)]: starting from
 * S_0 = text_init_scale * S_init, applies the frame write
 * S_t = (S_{t-1} Diag(alpha_t) + B_t)(I + A_t)^{-1}, as (S_{t-1} Diag(alpha_t)) N_t + J_t
 * over the scanned frames in increasing order and records vda_state_count()
 * states per head into `states` [H][count][d][d] float32 (states[h][0] = S_0).
 *  S_init = s_init [H][d][d] float32 when s_init != NULL, else S^T built from
 *  the text tokens in ws (zero when text_tokens == 0).
 *  ws must hold the output of vda_prepare_frames for the same desc.
 * With VDA_CHUNK_SCAN the same states come from C chunk steps
 * S <- S M_c + J_c; ws must then also hold the output of vda_compose_chunks,
 * which already applied alpha (the alpha argument is checked but not read). */
int vda_scan_fwd(const vda_desc* desc, const void* ws, const float* alpha, const float* s_init,
                 float* states, void* stream);

/* Reverse scan: the same recurrence over the scanned frames in decreasing
 * order, each frame with its own alpha_t; states[h][j] is the state after the
 * last j chunks (or frames when window == -1). */
int vda_scan_rev(const vda_desc* desc, const void* ws, const float* alpha, const float* s_init,
                 float* states, void* stream);

/* Both scans in one launch: the same work and results as vda_scan_fwd
 * (into states_fwd) and vda_scan_rev (into states_rev) with the same s_init,
 * run side by side on the GPU. */
int vda_scan_bidir(const vda_desc* desc, const void* ws, const float* alpha, const float* s_init,
                   float* states_fwd, float* states_rev, void* stream);

/* Readout [VDN 核心方法 para 1; 方法步骤详情 step (5)].  window >= 0: for a
 * scanned frame t of chunk c and each token,
 *   o = states_fwd[F(c)] (b_f * q) + states_rev[R(c)] (b_r * q),
 *   b_f = prod_{r=ws}^{t} alpha_r,  b_r = prod_{r=t}^{we} alpha_r
 * (b = 1 with VDA_NO_BRIDGE).  window == -1: o = states_fwd[t-anchors+1] q and
 * states_rev may be NULL.  Anchor frames get zero rows.
 *  q [H][T][U][d] in_dtype; out [H][T][U][d] out_dtype (every element written). */
int vda_readout(const vda_desc* desc, const void* q, const float* alpha, const float* states_fwd,
                const float* states_rev, void* out, void* stream);

/* The readout followed by the epilogue of the linear branch [VDN 方法步骤详情
 * step (5): the read is RMS-normalised and then passes a sigmoid gate;
 * VDN 核心方法 para 1: the linear branch is normalised before its gate].  For
 * every token of every scanned frame, over its d value channels c,
 *   y_c = o_c / sqrt(mean_c' o_c'^2 + eps) * norm_weight[h][c] * sigmoid(gate_c)
 * where o is what vda_readout computes from the same q, alpha and states.
 *  gate [H][T][U][d] logits in in_dtype (a per-channel gate projection of the
 *    layer input, computed by the caller); norm_weight [H][d] float32;
 *  eps > 0 and finite, else VDA_ERR_VALUE;
 *  out [H][T][U][d] out_dtype, every element written; anchor rows are zero.
 * The other arguments, layouts and errors are those of vda_readout. */
int vda_readout_gated(const vda_desc* desc, const void* q, const float* alpha, const float* states_fwd,
                      const float* states_rev, const void* gate, const float* norm_weight, float eps, void* out,
                      void* stream);

/* The softmax branch of the hybrid attention [VDN 核心方法 para 1;
 * 方法步骤详情 step (1)]: every query token of frame t attends, with
 *   o = softmax(q K^T * scale) V,
 * to the tokens of its visible frames and to all text tokens:
 *  - a frame of chunk c sees the frames of chunks c-w .. c+w (clipped to
 *    [0, C-1]) and the two anchor frames;
 *  - an anchor frame (0 or T-1) sees every frame.
 * q, k [H][T][U][d] and k_text [H][N_text][d] are bf16 (the projections
 * after the branch's QK normalisation and rotary encoding); v [H][T][U][d]
 * and v_text [H][N_text][d] are v_dtype, VDA_BF16 or VDA_F16 (f16 values
 * are used as given; bf16 ones are converted to f16 in the kernel, which
 * costs some throughput); out [H][T][U][d] out_dtype, every row written
 * (anchor rows included).
 * Needs in_dtype == VDA_BF16 (else VDA_ERR_DTYPE), d in {32, 64, 128} and
 * window >= 0 (else VDA_ERR_SHAPE), scale > 0 and finite (else
 * VDA_ERR_VALUE; 1/sqrt(d) is the usual choice).  VDA_PREP and VDA_NO_BRIDGE
 * do not apply.  k_text and v_text may be NULL when text_tokens == 0. */
int vda_softmax_branch(const vda_desc* desc, const void* q, const void* k, const void* v, const void* k_text,
                       const void* v_text, int32_t v_dtype, float scale, void* out, void* stream);

/* The whole path in one call: vda_prepare_frames, vda_compose_chunks (with
 * VDA_CHUNK_SCAN only), vda_scan_bidir (S_init =
 * S^T from the text tokens, or zero) and vda_readout, with the same
 * arguments, layouts and results as those calls made in that order on
 * `stream`; everything is enqueued on `stream` alone.  states_rev may be
 * NULL when window == -1 (the reverse scan is then skipped). */
int vda_forward(const vda_desc* desc, const void* q, const void* k, const void* v, const float* beta,
                const float* alpha, const void* k_text, const void* v_text, const float* beta_text,
                void* ws, size_t ws_bytes, float* states_fwd, float* states_rev, void* out,
                void* stream);

/* vda_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same path, kernels and results as vda_forward, with the workspace taken
 * from a device array the library holds, 64 MiB per device, from the first
 * use on a device until the process ends.  The call itself allocates
 * nothing.  Paths needing a larger workspace (vda_workspace_bytes(desc) >
 * 64 MiB, e.g. more than five heads of the H3-shaped layer) return
 * VDA_ERR_WORKSPACE before anything is enqueued.  status: NULL, or a device
 * int32 that receives the device status word (VDA_DEV_* bits) at the end of
 * the enqueued work.  Every call on one device shares that array, and it
 * keeps the last call's contents: calls that overlap on one device (on
 * different streams, or from different threads without ordering) race and
 * give undefined results.  The other arguments, layouts and errors are those
 * of vda_forward. */
int vda_forward_noalloc(const vda_desc* desc, const void* q, const void* k, const void* v, const float* beta,
                        const float* alpha, const void* k_text, const void* v_text, const float* beta_text,
                        float* states_fwd, float* states_rev, void* out, int32_t* status, void* stream);

/* Measurement aid (not part of the path): reads `bytes` (a multiple of 16)
 * of device memory at `src` with 16-byte loads in `blocks` workgroups of 256
 * threads and writes one word per workgroup to sink [blocks] (device
 * uint32).  Timed around a large buffer it gives the read bandwidth a plain
 * streaming kernel reaches on the device, the practical ceiling of the
 * bandwidth-bound kernels of the path. */
int vda_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, void* stream);

/* Synchronises `stream`, then copies the device status word of `ws` into
 * *flags (VDA_DEV_* bits; 0 = no fault).  For tests and diagnostics. */
int vda_device_status(const vda_desc* desc, const void* ws, void* stream, int32_t* flags);

/* Static description of a return code. */
const char* vda_status_string(int code);

/* Message of the last failed call on this thread ("" if none). */
const char* vda_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VDA_H */
