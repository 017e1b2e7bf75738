// libvda C ABI: argument validation, index maps, workspace sizing and
// kernel launches.  All validation happens on the host before anything is
// enqueued, so it is testable without a GPU.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cmath>
#include <mutex>

#include "vda.h"
#include "vda_common.h"
#include "vda_kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_last_error[0] = '\0';
  return VDA_OK;
}

struct Shape {
  int H, T, U, d, P, a, n, C, w, Nt, n_eff, count;
  bool chunked;  // VDA_CHUNK_SCAN
  bool sana;     // VDA_SANA_WM
  bool newton;   // VDA_NEWTON
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Host-side validation of a descriptor; fills the derived sizes.
int check_desc(const vda_desc* desc, Shape* s) {
  if (!desc) return fail(VDA_ERR_NULL, "desc is NULL");
  const vda_desc& q = *desc;
  if (q.heads < 0) return fail(VDA_ERR_SHAPE, "heads = %d < 0", q.heads);
  if (q.tokens < 0) return fail(VDA_ERR_SHAPE, "tokens = %d < 0", q.tokens);
  if (q.d_k != q.d_v) return fail(VDA_ERR_SHAPE, "d_k (%d) != d_v (%d)", q.d_k, q.d_v);
  if (q.d_k != 16 && q.d_k != 32 && q.d_k != 64 && q.d_k != 128)
    return fail(VDA_ERR_SHAPE, "d = %d is not one of 16, 32, 64, 128", q.d_k);
  if (q.chunk < 1) return fail(VDA_ERR_SHAPE, "chunk = %d < 1", q.chunk);
  if (q.anchors != 0 && q.anchors != 1) return fail(VDA_ERR_SHAPE, "anchors = %d (0 or 1)", q.anchors);
  if (q.frames < 2 * q.anchors || q.frames < 0)
    return fail(VDA_ERR_SHAPE, "frames = %d < 2 * anchors", q.frames);
  if (q.window < -1) return fail(VDA_ERR_SHAPE, "window = %d < -1", q.window);
  if (q.text_tokens < 0) return fail(VDA_ERR_SHAPE, "text_tokens = %d < 0", q.text_tokens);
  if (q.in_dtype != VDA_F32 && q.in_dtype != VDA_BF16)
    return fail(VDA_ERR_DTYPE, "in_dtype = %d (VDA_F32 or VDA_BF16)", q.in_dtype);
  if (q.out_dtype != VDA_F32 && q.out_dtype != VDA_BF16 && q.out_dtype != VDA_F16)
    return fail(VDA_ERR_DTYPE, "out_dtype = %d (VDA_F32, VDA_BF16 or VDA_F16)", q.out_dtype);
  if (!(q.text_init_scale == q.text_init_scale)) return fail(VDA_ERR_SHAPE, "text_init_scale is NaN");
  if (q.flags & ~(uint32_t)(VDA_NO_BRIDGE | VDA_PREP | VDA_CHUNK_SCAN | VDA_SANA_WM | VDA_NEWTON))
    return fail(VDA_ERR_SHAPE, "unknown flags 0x%x", q.flags);
  if ((q.flags & VDA_SANA_WM) && (q.flags & VDA_NEWTON))
    return fail(VDA_ERR_SHAPE, "VDA_SANA_WM has no inverse for VDA_NEWTON to form");
  if ((q.flags & VDA_SANA_WM) && (q.flags & VDA_CHUNK_SCAN))
    return fail(VDA_ERR_SHAPE, "VDA_SANA_WM and VDA_CHUNK_SCAN cannot be combined");
  if ((q.flags & VDA_CHUNK_SCAN) && q.window < 0)
    return fail(VDA_ERR_SHAPE, "VDA_CHUNK_SCAN needs window >= 0 (states at chunk boundaries)");
  s->H = q.heads;
  s->T = q.frames;
  s->U = q.tokens;
  s->d = q.d_k;
  s->P = q.chunk;
  s->a = q.anchors;
  s->n = q.frames - 2 * q.anchors;
  s->C = (s->n + s->P - 1) / s->P;
  s->w = q.window;
  s->Nt = q.text_tokens;
  s->n_eff = s->n + (s->Nt > 0 ? 1 : 0);
  if (s->w >= 0 && s->n % s->P != 0)
    return fail(VDA_ERR_SHAPE, "windowed readout needs n %% chunk == 0 (n = %d, chunk = %d)", s->n, s->P);
  s->count = (s->w >= 0 ? s->C : s->n) + 1;
  s->chunked = (q.flags & VDA_CHUNK_SCAN) != 0;
  s->sana = (q.flags & VDA_SANA_WM) != 0;
  s->newton = (q.flags & VDA_NEWTON) != 0;
  // 64-bit sizes must not overflow and grids must fit
  const double elems = (double)s->H * s->T * (double)s->U * s->d;
  if (elems > 9.0e15) return fail(VDA_ERR_SHAPE, "tensor too large");
  if ((double)s->H * s->n_eff > 2.0e9 || (double)s->H * s->T > 2.0e9) return fail(VDA_ERR_SHAPE, "grid too large");
  return VDA_OK;
}

size_t ws_frames_bytes(const Shape& s) {
  return vda::kWsHeader + (size_t)s.H * s.n_eff * vda::ws_slot_floats(s.d) * sizeof(float);
}

// the chunk maps follow the frame slots: [H][2 directions][C] x 4 d^2 bytes
size_t ws_bytes(const Shape& s) {
  return ws_frames_bytes(s) + (s.chunked ? (size_t)s.H * 2 * s.C * 4 * s.d * s.d : 0);
}

// One-time check per device that it is a gfx950 GPU.
int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return fail(VDA_ERR_DEVICE, "no HIP device available");
  static std::mutex mu;
  static int known[64];  // 0 unknown, 1 ok, -1 bad
  if (dev < 0 || dev >= 64) return fail(VDA_ERR_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (known[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(VDA_ERR_DEVICE, "hipGetDeviceProperties failed");
    known[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    if (known[dev] < 0) return fail(VDA_ERR_DEVICE, "device %d is %s, libvda needs gfx950", dev, prop.gcnArchName);
  }
  if (known[dev] < 0) return fail(VDA_ERR_DEVICE, "device %d is not gfx950", dev);
  return VDA_OK;
}

int launch_status() {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(VDA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

const char* vda_status_string(int code) {
  switch (code) {
    case VDA_OK: return "ok";
    case VDA_ERR_NULL: return "null pointer";
    case VDA_ERR_SHAPE: return "invalid shape";
    case VDA_ERR_DTYPE: return "unsupported dtype";
    case VDA_ERR_ALIGN: return "misaligned pointer";
    case VDA_ERR_WORKSPACE: return "workspace too small";
    case VDA_ERR_HIP: return "HIP error";
    case VDA_ERR_DEVICE: return "no usable gfx950 device";
    case VDA_ERR_VALUE: return "argument out of range";
    default: return "unknown status";
  }
}

const char* vda_last_error(void) { return g_last_error; }

int vda_workspace_bytes(const vda_desc* desc, size_t* bytes) {
  Shape s;
  int rc = check_desc(desc, &s);
  if (rc) return rc;
  if (!bytes) return fail(VDA_ERR_NULL, "bytes is NULL");
  *bytes = ws_bytes(s);
  return ok();
}

int vda_state_count(const vda_desc* desc, int32_t* count) {
  Shape s;
  int rc = check_desc(desc, &s);
  if (rc) return rc;
  if (!count) return fail(VDA_ERR_NULL, "count is NULL");
  *count = s.count;
  return ok();
}

int vda_index_map(const vda_desc* desc, int32_t* chunk_rows, int32_t* frame_chunk) {
  Shape s;
  int rc = check_desc(desc, &s);
  if (rc) return rc;
  const int w = s.w < 0 ? 0 : s.w;
  if (chunk_rows) {
    for (int c = 0; c < s.C; ++c) {
      const vda::ChunkWindow cw = vda::chunk_window(c, s.C, w, s.P, s.a, s.n);
      int32_t* r = chunk_rows + 7 * (size_t)c;
      r[0] = c;
      r[1] = cw.lo;
      r[2] = cw.hi;
      r[3] = cw.ws;
      r[4] = cw.we;
      r[5] = cw.F;
      r[6] = cw.R;
    }
  }
  if (frame_chunk) {
    for (int t = 0; t < s.T; ++t) frame_chunk[t] = vda::frame_chunk_of(t, s.a, s.n, s.P);
  }
  return ok();
}

int vda_index_map_device(const vda_desc* desc, int32_t* chunk_rows, int32_t* frame_chunk, void* stream) {
  Shape s;
  int rc = check_desc(desc, &s);
  if (rc) return rc;
  if ((!chunk_rows && s.C > 0) || (!frame_chunk && s.T > 0))
    return fail(VDA_ERR_NULL, "chunk_rows or frame_chunk is NULL");
  if (!aligned16(chunk_rows) || !aligned16(frame_chunk))
    return fail(VDA_ERR_ALIGN, "chunk_rows and frame_chunk need 16-byte alignment");
  rc = check_device();
  if (rc) return rc;
  vda::launch_index_map(s.C, s.T, s.w < 0 ? 0 : s.w, s.P, s.a, s.n, chunk_rows, frame_chunk,
                        static_cast<hipStream_t>(stream));
  return launch_status();
}

}  // extern "C"

namespace {

// Validation + argument blocks of the individual steps (host only).
int prep_args(const vda_desc* desc, const void* k, const void* v, const float* beta, const void* k_text,
              const void* v_text, const float* beta_text, void* ws, size_t ws_size, Shape& s,
              vda::PrepArgs& a) {
  int rc = check_desc(desc, &s);
  if (rc) return rc;
  const bool need_video = (size_t)s.H * s.n * s.U > 0;
  if (need_video && (!k || !v || !beta)) return fail(VDA_ERR_NULL, "k, v or beta is NULL");
  if (s.Nt > 0 && s.H > 0 && (!k_text || !v_text || !beta_text))
    return fail(VDA_ERR_NULL, "k_text, v_text or beta_text is NULL with text_tokens = %d", s.Nt);
  if (!ws) return fail(VDA_ERR_NULL, "ws is NULL");
  if (ws_size < ws_bytes(s)) return fail(VDA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_size, ws_bytes(s));
  if (!aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(k_text) || !aligned16(v_text) ||
      !aligned16(beta_text) || ((uintptr_t)ws & 255u))
    return fail(VDA_ERR_ALIGN, "k, v, beta, k_text, v_text, beta_text need 16-byte and ws 256-byte alignment");
  a.k = k;
  a.v = v;
  a.beta = beta;
  a.kt = k_text;
  a.vt = v_text;
  a.bt = beta_text;
  a.status = static_cast<int*>(ws);
  a.frames = reinterpret_cast<float*>(static_cast<char*>(ws) + vda::kWsHeader);
  a.H = s.H;
  a.T = s.T;
  a.U = s.U;
  a.a = s.a;
  a.n = s.n;
  a.n_eff = s.n_eff;
  a.Nt = s.Nt;
  a.s0 = 0;
  a.cnt = s.n_eff;
  a.prep = (desc->flags & VDA_PREP) ? 1 : 0;
  return VDA_OK;
}

int scan_args(const vda_desc* desc, const void* ws, const float* alpha, const float* s_init, float* states,
              int reverse, Shape& s, vda::ScanArgs& a, bool need_states = true) {
  int rc = check_desc(desc, &s);
  if (rc) return rc;
  if (!ws) return fail(VDA_ERR_NULL, "ws is NULL");
  if (need_states && !states) return fail(VDA_ERR_NULL, "states is NULL");
  if (s.H * (size_t)s.n > 0 && !alpha) return fail(VDA_ERR_NULL, "alpha is NULL");
  if (!aligned16(alpha) || !aligned16(s_init) || !aligned16(states) || ((uintptr_t)ws & 255u))
    return fail(VDA_ERR_ALIGN, "alpha, s_init, states need 16-byte and ws 256-byte alignment");
  a.frames = reinterpret_cast<const float*>(static_cast<const char*>(ws) + vda::kWsHeader);
  a.status = static_cast<int*>(const_cast<void*>(ws));
  a.alpha = alpha;
  a.s_init = s_init;
  a.states = states;
  a.H = s.H;
  a.T = s.T;
  a.a = s.a;
  a.n = s.n;
  a.n_eff = s.n_eff;
  a.count = s.count;
  a.every = s.w >= 0 ? s.P : 1;
  a.reverse = reverse;
  a.use_text = s.Nt > 0;
  a.scale = desc->text_init_scale;
  a.prep = (desc->flags & VDA_PREP) ? 1 : 0;
  a.chunks = const_cast<char*>(static_cast<const char*>(ws)) + ws_frames_bytes(s);
  a.C = s.C;
  a.P = s.P;
  return VDA_OK;
}

int scan_mode(const Shape& s) {
  if (s.sana) return vda::kSanaScan;
  if (s.chunked) return vda::kChunkScan;
  return s.newton ? vda::kFrameScanB : vda::kFrameScan;
}

// Everything the scans read from the workspace: N_t and J_t from the fused
// statistics + factorisation kernel; for the comparators, the statistics and
// then the Newton-iteration inverse (N_t, with B_t) or the SANA-WM transition
// and injection.  The device status word is cleared first.
void launch_prepare(const Shape& s, const vda::PrepArgs& a, bool in_f32, hipStream_t st) {
  vda::launch_clear_status(a.status, st);
  if (s.sana) {
    vda::launch_stats(a, s.d, in_f32, st);
    vda::launch_sana(a, s.d, st);
  } else if (s.newton) {
    vda::launch_stats(a, s.d, in_f32, st);
    vda::launch_ns(a, s.d, st);
  } else {
    vda::launch_frame(a, s.d, in_f32, st);
  }
}

int read_args(const vda_desc* desc, const void* q, const float* alpha, const float* states_fwd,
              const float* states_rev, void* out, Shape& s, vda::ReadArgs& a, bool& any) {
  int rc = check_desc(desc, &s);
  if (rc) return rc;
  any = (size_t)s.H * s.T * s.U > 0;
  if (any && !out) return fail(VDA_ERR_NULL, "out is NULL");
  if (any && s.n > 0) {
    if (!q || !states_fwd) return fail(VDA_ERR_NULL, "q or states_fwd is NULL");
    if (!alpha && s.w >= 0) return fail(VDA_ERR_NULL, "alpha is NULL");
    if (s.w >= 0 && !states_rev) return fail(VDA_ERR_NULL, "states_rev is NULL with window >= 0");
  }
  if (!aligned16(q) || !aligned16(alpha) || !aligned16(states_fwd) || !aligned16(states_rev) || !aligned16(out))
    return fail(VDA_ERR_ALIGN, "q, alpha, states, out need 16-byte alignment");
  a.q = q;
  a.alpha = alpha;
  a.sf = states_fwd;
  a.sr = states_rev;
  a.out = out;
  a.H = s.H;
  a.T = s.T;
  a.U = s.U;
  a.a = s.a;
  a.n = s.n;
  a.P = s.P;
  a.C = s.C;
  a.w = s.w;
  a.count = s.count;
  a.bridge = (desc->flags & VDA_NO_BRIDGE) ? 0 : 1;
  a.prep = (desc->flags & VDA_PREP) ? 1 : 0;
  a.gate = nullptr;
  a.normw = nullptr;
  a.eps = 0.f;
  return VDA_OK;
}

}  // namespace

extern "C" {

int vda_prepare_frames(const vda_desc* desc, const void* k, const void* v, const float* beta,
                       const void* k_text, const void* v_text, const float* beta_text, void* ws,
                       size_t ws_size, void* stream) {
  Shape s;
  vda::PrepArgs a;
  int rc = prep_args(desc, k, v, beta, k_text, v_text, beta_text, ws, ws_size, s, a);
  if (rc) return rc;
  rc = check_device();
  if (rc) return rc;
  launch_prepare(s, a, desc->in_dtype == VDA_F32, static_cast<hipStream_t>(stream));
  return launch_status();
}

int vda_scan_fwd(const vda_desc* desc, const void* ws, const float* alpha, const float* s_init, float* states,
                 void* stream) {
  Shape s;
  vda::ScanArgs a;
  int rc = scan_args(desc, ws, alpha, s_init, states, 0, s, a);
  if (rc) return rc;
  rc = check_device();
  if (rc) return rc;
  vda::ScanPair p = {{a, a}, 1, scan_mode(s), s.newton};
  vda::launch_scan(p, s.d, static_cast<hipStream_t>(stream));
  return launch_status();
}

int vda_scan_rev(const vda_desc* desc, const void* ws, const float* alpha, const float* s_init, float* states,
                 void* stream) {
  Shape s;
  vda::ScanArgs a;
  int rc = scan_args(desc, ws, alpha, s_init, states, 1, s, a);
  if (rc) return rc;
  rc = check_device();
  if (rc) return rc;
  vda::ScanPair p = {{a, a}, 1, scan_mode(s), s.newton};
  vda::launch_scan(p, s.d, static_cast<hipStream_t>(stream));
  return launch_status();
}

int vda_compose_chunks(const vda_desc* desc, void* ws, size_t ws_size, const float* alpha, void* stream) {
  Shape s;
  vda::ScanPair p;
  int rc = scan_args(desc, ws, alpha, nullptr, nullptr, 0, s, p.dir[0], false);
  if (rc) return rc;
  if (!s.chunked) return fail(VDA_ERR_SHAPE, "vda_compose_chunks needs VDA_CHUNK_SCAN in desc.flags");
  if (ws_size < ws_bytes(s)) return fail(VDA_ERR_WORKSPACE, "workspace %zu < %zu bytes", ws_size, ws_bytes(s));
  scan_args(desc, ws, alpha, nullptr, nullptr, 1, s, p.dir[1], false);
  rc = check_device();
  if (rc) return rc;
  p.ndir = 2;
  p.mode = vda::kCompose;
  p.bform = s.newton;
  vda::launch_scan(p, s.d, static_cast<hipStream_t>(stream));
  return launch_status();
}

int vda_scan_bidir(const vda_desc* desc, const void* ws, const float* alpha, const float* s_init,
                   float* states_fwd, float* states_rev, void* stream) {
  Shape s;
  vda::ScanPair p;
  int rc = scan_args(desc, ws, alpha, s_init, states_fwd, 0, s, p.dir[0]);
  if (rc) return rc;
  if ((rc = scan_args(desc, ws, alpha, s_init, states_rev, 1, s, p.dir[1]))) return rc;
  rc = check_device();
  if (rc) return rc;
  p.ndir = 2;
  p.mode = scan_mode(s);
  p.bform = s.newton;
  vda::launch_scan(p, s.d, static_cast<hipStream_t>(stream));
  return launch_status();
}

int vda_readout(const vda_desc* desc, const void* q, const float* alpha, const float* states_fwd,
                const float* states_rev, void* out, void* stream) {
  Shape s;
  vda::ReadArgs a;
  bool any = false;
  int rc = read_args(desc, q, alpha, states_fwd, states_rev, out, s, a, any);
  if (rc) return rc;
  rc = check_device();
  if (rc) return rc;
  if (!any) return ok();
  vda::launch_readout(a, s.d, desc->in_dtype, desc->out_dtype, static_cast<hipStream_t>(stream));
  return launch_status();
}

int vda_readout_gated(const vda_desc* desc, const void* q, const float* alpha, const float* states_fwd,
                      const float* states_rev, const void* gate, const float* norm_weight, float eps, void* out,
                      void* stream) {
  Shape s;
  vda::ReadArgs a;
  bool any = false;
  int rc = read_args(desc, q, alpha, states_fwd, states_rev, out, s, a, any);
  if (rc) return rc;
  if (any && s.n > 0 && (!gate || !norm_weight)) return fail(VDA_ERR_NULL, "gate or norm_weight is NULL");
  if (!aligned16(gate) || !aligned16(norm_weight)) return fail(VDA_ERR_ALIGN, "gate, norm_weight need 16-byte alignment");
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(VDA_ERR_VALUE, "eps must be positive and finite");
  rc = check_device();
  if (rc) return rc;
  if (!any) return ok();
  a.gate = gate;
  a.normw = norm_weight;
  a.eps = eps;
  vda::launch_readout_gated(a, s.d, desc->in_dtype, desc->out_dtype, static_cast<hipStream_t>(stream));
  return launch_status();
}

int vda_softmax_branch(const vda_desc* desc, const void* q, const void* k, const void* v, const void* k_text,
                       const void* v_text, int32_t v_dtype, float scale, void* out, void* stream) {
  Shape s;
  int rc = check_desc(desc, &s);
  if (rc) return rc;
  if (desc->in_dtype != VDA_BF16) return fail(VDA_ERR_DTYPE, "the softmax branch needs bf16 q and k");
  if (v_dtype != VDA_BF16 && v_dtype != VDA_F16)
    return fail(VDA_ERR_DTYPE, "v_dtype = %d (VDA_BF16 or VDA_F16)", v_dtype);
  if (s.d == 16) return fail(VDA_ERR_SHAPE, "the softmax branch needs d in {32, 64, 128}");
  if (s.w < 0) return fail(VDA_ERR_SHAPE, "the softmax branch needs window >= 0");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(VDA_ERR_VALUE, "scale must be positive and finite");
  const bool any = (size_t)s.H * s.T * s.U > 0;
  if (any && (!q || !k || !v || !out)) return fail(VDA_ERR_NULL, "q, k, v or out is NULL");
  if (any && s.Nt > 0 && (!k_text || !v_text)) return fail(VDA_ERR_NULL, "k_text or v_text is NULL with text_tokens = %d", s.Nt);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(k_text) || !aligned16(v_text) || !aligned16(out))
    return fail(VDA_ERR_ALIGN, "q, k, v, k_text, v_text, out need 16-byte alignment");
  rc = check_device();
  if (rc) return rc;
  if (!any) return ok();
  vda::AttnArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.kt = k_text;
  a.vt = v_text;
  a.out = out;
  a.H = s.H;
  a.T = s.T;
  a.U = s.U;
  a.a = s.a;
  a.P = s.P;
  a.C = s.C;
  a.w = s.w;
  a.Nt = s.Nt;
  a.scale = scale;
  a.v_f16 = v_dtype == VDA_F16;
  const int qb = 256;  // queries per workgroup (the attention kernel's kQB)
  a.anchor_tiles = s.a ? (s.U + qb - 1) / qb : 0;
  a.chunk_tiles = (s.P * s.U + qb - 1) / qb;
  a.tiles_per_head = 2 * a.anchor_tiles + s.C * a.chunk_tiles;
  if ((double)s.H * a.tiles_per_head > 2.0e9) return fail(VDA_ERR_SHAPE, "grid too large");
  vda::launch_attn(a, s.d, desc->out_dtype, static_cast<hipStream_t>(stream));
  return launch_status();
}

}  // extern "C"

namespace {

// The whole path on one stream (vda_forward, and vda_forward_noalloc with
// its own workspace).
int forward_impl(const vda_desc* desc, const void* q, const void* k, const void* v, const float* beta,
                 const float* alpha, const void* k_text, const void* v_text, const float* beta_text, void* ws,
                 size_t ws_size, float* states_fwd, float* states_rev, void* out, void* stream) {
  Shape s;
  vda::PrepArgs pa;
  vda::ScanPair sp;
  vda::ReadArgs qa;
  bool any = false;
  int rc = prep_args(desc, k, v, beta, k_text, v_text, beta_text, ws, ws_size, s, pa);
  if (rc) return rc;
  const bool rev = states_rev != nullptr || s.w >= 0;
  if ((rc = scan_args(desc, ws, alpha, nullptr, states_fwd, 0, s, sp.dir[0]))) return rc;
  sp.dir[1] = sp.dir[0];
  if (rev && (rc = scan_args(desc, ws, alpha, nullptr, states_rev, 1, s, sp.dir[1]))) return rc;
  sp.ndir = rev ? 2 : 1;
  if ((rc = read_args(desc, q, alpha, states_fwd, states_rev, out, s, qa, any))) return rc;
  if ((rc = check_device())) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  sp.bform = s.newton;
  launch_prepare(s, pa, desc->in_dtype == VDA_F32, st);
  if (s.chunked) {
    vda::ScanPair cp = sp;  // both directions' chunk maps in one launch
    cp.dir[1] = sp.dir[0];
    cp.dir[1].reverse = 1;
    cp.ndir = 2;
    cp.mode = vda::kCompose;
    vda::launch_scan(cp, s.d, st);
  }
  sp.mode = scan_mode(s);
  vda::launch_scan(sp, s.d, st);  // both directions in one launch
  if (any) vda::launch_readout(qa, s.d, desc->in_dtype, desc->out_dtype, st);
  return launch_status();
}

// Workspace of vda_forward_noalloc: a file-scope device array, one copy per
// device, held from the library's load until the process ends.  In host
// code `scratch` names a host-side stand-in, so its device address is taken
// once per device with hipGetSymbolAddress (with that device current) and
// only that address is handed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_addr[64];  // device address of `scratch`, per device index

int scratch_address(void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(VDA_ERR_DEVICE, "no usable HIP device for the no-alloc workspace");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(VDA_ERR_HIP, "hipGetSymbolAddress of the no-alloc workspace failed: %s", hipGetErrorString(e));
    g_scratch_addr[dev] = p;
  }
  *addr = g_scratch_addr[dev];
  return VDA_OK;
}

// Streams n16 16-byte words of src through the vector memory path (eight
// independent loads in flight per thread) and writes one word per workgroup
// to sink, so that the loads cannot be dropped.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4* __restrict__ src, size_t n16, uint32_t* sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  uint32_t x = 0;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = src[i + j * stride];
#pragma unroll
    for (int j = 0; j < 8; ++j) x ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int t = 0; t < 256; ++t) r ^= red[t];
    sink[blockIdx.x] = r;
  }
}

}  // namespace

extern "C" {

int vda_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks, void* stream) {
  if (!src || !sink) return fail(VDA_ERR_NULL, "src or sink is NULL");
  if (!aligned16(src) || (bytes & 15u)) return fail(VDA_ERR_ALIGN, "src and bytes need 16-byte alignment");
  if (blocks < 1) return fail(VDA_ERR_VALUE, "blocks = %d < 1", blocks);
  int rc = check_device();
  if (rc) return rc;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(src), bytes / 16, sink);
  return launch_status();
}

int vda_forward(const vda_desc* desc, const void* q, const void* k, const void* v, const float* beta,
                const float* alpha, const void* k_text, const void* v_text, const float* beta_text, void* ws,
                size_t ws_size, float* states_fwd, float* states_rev, void* out, void* stream) {
  return forward_impl(desc, q, k, v, beta, alpha, k_text, v_text, beta_text, ws, ws_size, states_fwd, states_rev,
                      out, stream);
}

int vda_forward_noalloc(const vda_desc* desc, const void* q, const void* k, const void* v, const float* beta,
                        const float* alpha, const void* k_text, const void* v_text, const float* beta_text,
                        float* states_fwd, float* states_rev, void* out, int32_t* status, void* stream) {
  Shape s;
  int rc = check_desc(desc, &s);
  if (rc) return rc;
  if (ws_bytes(s) > kScratchBytes)
    return fail(VDA_ERR_WORKSPACE, "the path needs %zu bytes of workspace; vda_forward_noalloc holds at most %zu",
                ws_bytes(s), kScratchBytes);
  if (!aligned16(status)) return fail(VDA_ERR_ALIGN, "status needs 16-byte alignment");
  if ((rc = check_device())) return rc;
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  rc = forward_impl(desc, q, k, v, beta, alpha, k_text, v_text, beta_text, ws, kScratchBytes, states_fwd, states_rev,
                    out, stream);
  if (rc) return rc;
  if (status) vda::launch_copy_status(static_cast<const int*>(ws), status, static_cast<hipStream_t>(stream));
  return launch_status();
}

int vda_device_status(const vda_desc* desc, const void* ws, void* stream, int32_t* flags) {
  Shape s;
  int rc = check_desc(desc, &s);
  if (rc) return rc;
  if (!ws || !flags) return fail(VDA_ERR_NULL, "ws or flags is NULL");
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (hipStreamSynchronize(st) != hipSuccess) return fail(VDA_ERR_HIP, "hipStreamSynchronize failed");
  int32_t v = 0;
  if (hipMemcpy(&v, ws, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess)
    return fail(VDA_ERR_HIP, "reading the status word failed");
  *flags = v;
  return ok();
}

}  // extern "C"
