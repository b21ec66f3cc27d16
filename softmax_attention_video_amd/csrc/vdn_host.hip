// C-ABI of the VDN attention library: argument checks, workspace layout and
// launch sequencing.  Every check runs on the host before the first HIP call.
#include "../../include/vdn.h"
#include "gemm_nt.h"
#include "vdn_internal.h"
#include "window_items.h"

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

namespace {

thread_local char g_err[512] = "";

vdn_status fail(vdn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

#define VDN_HIP(expr)                                                                   \
  do {                                                                                  \
    hipError_t e_ = (expr);                                                             \
    if (e_ != hipSuccess)                                                               \
      return fail(VDN_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(e_));          \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Per-thread kernel timer (see vdn_timer_enable).
struct KernelTimer {
  hipEvent_t* ev = nullptr;
  int cap = 0, used = 0;
};
thread_local KernelTimer g_timer;

hipError_t timer_mark(hipStream_t s, bool begin) {
  if (!g_timer.ev || g_timer.used >= g_timer.cap) return hipSuccess;
  hipError_t e = hipEventRecord(g_timer.ev[2 * g_timer.used + (begin ? 0 : 1)], s);
  if (!begin) ++g_timer.used;
  return e;
}

// Per-thread, per-device side stream and fork/join events for running the
// VDA linear branch concurrently with the window Softmax.  Created on first
// use at default priority; they live until the thread exits.
struct SideStream {
  int device = -1;
  hipStream_t stream = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
thread_local SideStream g_side[16];

hipError_t side_stream(SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 16) return hipErrorInvalidDevice;
  SideStream& ss = g_side[dev];
  if (!ss.stream) {
    if ((e = hipStreamCreateWithFlags(&ss.stream, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming)) != hipSuccess) return e;
    ss.device = dev;
  }
  *out = &ss;
  return hipSuccess;
}

// Workspace carve-up (offsets in bytes, each 256-aligned).  Each entry point
// takes only the regions it uses; vdn_attn_fwd takes them all, with the
// branch outputs Ohat_s, Ohat_l last so that a caller who passes its own
// buffers for them needs no room for them.
struct Layout {
  size_t vt, wt0, wt1, Tf, Uf, St, Tc, Uc, Pf, Pr;
  size_t mxa, mxas, mxw, mxws;   // MX-FP8 merge operands: codes and scales of A and W^T
  size_t ohs, ohl;
  size_t total;
};

enum class Entry { Attn, Scan, Softmax, Merge };

// mx: the merge runs in MX-FP8 (vdn_params.merge_mxfp8 on the bf16 path).
Layout make_layout(const vdn::Geometry& g, int Dm, vdn_dtype dt, bool mx, Entry e) {
  const size_t es = dt == VDN_BF16 ? 2 : 4;
  const size_t BH = (size_t)g.B * g.H, DD = (size_t)g.D * g.D;
  const size_t M = (size_t)g.B * g.L, K2 = 2 * (size_t)g.H * g.D;
  const bool attn = e == Entry::Attn;
  const bool sm = attn || e == Entry::Softmax;
  const bool scan = attn || e == Entry::Scan;
  const bool merge = attn || e == Entry::Merge;
  const bool bf16 = dt == VDN_BF16;
  // chunk maps exist only where the chunk-composed scan runs (d = 16, 32);
  // d = 64, 128 scan the frame maps directly
  const bool compose = g.D != 64 && g.D != 128;
  Layout l{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += align256(bytes); return r; };
  l.vt = take(sm && bf16 && vdn::window_softmax_mfma_ok(g) ? BH * (size_t)vdn::softmax_vt_pitch(g) * g.D * es : 0);
  l.wt0 = take(merge && bf16 ? (size_t)g.H * g.D * Dm * es : 0);
  l.wt1 = take(merge && bf16 ? (size_t)g.H * g.D * Dm * es : 0);
  l.Tf = take(scan ? BH * g.F * DD * 4 : 0);
  l.Uf = take(scan ? BH * g.F * DD * 4 : 0);
  l.St = take(scan ? BH * DD * 4 : 0);
  l.Tc = take(scan && compose ? BH * 2 * g.C * DD * 4 : 0);
  l.Uc = take(scan && compose ? BH * 2 * g.C * DD * 4 : 0);
  l.Pf = take(attn ? BH * (g.C + 1) * DD * 4 : 0);
  l.Pr = take(attn ? BH * (g.C + 1) * DD * 4 : 0);
  l.mxa = take(merge && mx ? M * K2 : 0);
  l.mxas = take(merge && mx ? M * K2 / 32 : 0);
  l.mxw = take(merge && mx ? (size_t)Dm * K2 : 0);
  l.mxws = take(merge && mx ? (size_t)Dm * K2 / 32 : 0);
  l.ohs = take(attn ? BH * g.L * g.D * es : 0);
  l.ohl = take(attn ? BH * g.L * g.D * es : 0);
  l.total = o;
  return l;
}

// Workspace of the Softmax backward: g_s * dOhat in head-major order and Dq.
struct BwdLayout {
  size_t dohm, Dq, total;
};

BwdLayout bwd_layout(const vdn::Geometry& g, vdn_dtype dt) {
  const size_t es = dt == VDN_BF16 ? 2 : 4;
  const size_t rows = (size_t)g.B * g.H * g.L;
  BwdLayout l{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += align256(bytes); return r; };
  l.dohm = take(rows * g.D * es);
  l.Dq = take(rows * 4);
  l.total = o;
  return l;
}

// Workspace of the linear-branch backward: the forward recompute (frame maps,
// inverses, chunk maps, boundary states) and the adjoint buffers (fp32).
struct VdaBwdLayout {
  size_t Tf, Uf, Xf, St, Tc, Uc, Pf, Pr, G, Dbr, dDbr, dgp, dP, mu, Sst, Zst, ZT, Rscr, total;
};

VdaBwdLayout vda_bwd_layout(const vdn::Geometry& g) {
  const size_t BH = (size_t)g.B * g.H, DD = (size_t)g.D * g.D, F = g.F, C = g.C;
  VdaBwdLayout l{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += align256(bytes); return r; };
  l.Tf = take(BH * F * DD * 4);
  l.Uf = take(BH * F * DD * 4);
  l.Xf = take(BH * (F + 1) * DD * 4);
  l.St = take(BH * DD * 4);
  l.Tc = take(BH * 2 * C * DD * 4);
  l.Uc = take(BH * 2 * C * DD * 4);
  l.Pf = take(BH * (C + 1) * DD * 4);
  l.Pr = take(BH * (C + 1) * DD * 4);
  l.G = take(BH * F * DD * 4);
  l.Dbr = take(BH * 2 * F * g.D * 4);
  l.dDbr = take(BH * 2 * F * g.D * 4);
  l.dgp = take(BH * F * g.D * 4);
  l.dP = take(BH * 2 * (C + 1) * DD * 4);
  l.mu = take(BH * 2 * (C + 1) * DD * 4);
  l.Sst = take(BH * 2 * (F + 1) * DD * 4);
  l.Zst = take(BH * 2 * F * DD * 4);
  l.ZT = take(BH * DD * 4);
  l.Rscr = take(BH * F * g.D * 4);
  l.total = o;
  return l;
}

bool use_mx(const vdn_params* p, vdn_dtype dt) { return p->merge_mxfp8 == 1 && dt == VDN_BF16; }

vdn_params defaults() {
  vdn_params p;
  p.softmax_scale = 0.f;
  p.rms_eps = 1e-6f;
  p.text_init_scale = 0.5f;
  p.chunk_frames = 5;
  p.window_chunks = 1;
  p.anchors = 1;
  p.text_softmax = 0;
  p.merge_mxfp8 = 0;
  return p;
}

// Shape / parameter checks shared by all entry points.
vdn_status check_geometry(const vdn_dims* d, const vdn_params* p, vdn_dtype dt, vdn::Geometry* g) {
  if (!d) return fail(VDN_ERR_INVALID_ARG, "dims is NULL");
  if (!p) return fail(VDN_ERR_INVALID_ARG, "params is NULL");
  if (dt != VDN_F32 && dt != VDN_BF16) return fail(VDN_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  if (d->B < 1 || d->H < 1) return fail(VDN_ERR_INVALID_ARG, "B=%d H=%d must be >= 1", d->B, d->H);
  if (d->F < 2) return fail(VDN_ERR_INVALID_ARG, "F=%d must be >= 2", d->F);
  if (d->N < 1) return fail(VDN_ERR_INVALID_ARG, "N=%d must be >= 1", d->N);
  if (d->T < 0) return fail(VDN_ERR_INVALID_ARG, "T=%d must be >= 0", d->T);
  if (p->chunk_frames < 1) return fail(VDN_ERR_INVALID_ARG, "chunk_frames=%d must be >= 1", p->chunk_frames);
  if (p->window_chunks < 0) return fail(VDN_ERR_INVALID_ARG, "window_chunks=%d must be >= 0", p->window_chunks);
  if (p->anchors != 0 && p->anchors != 1) return fail(VDN_ERR_INVALID_ARG, "anchors=%d must be 0 or 1", p->anchors);
  if (p->text_softmax != 0 && p->text_softmax != 1)
    return fail(VDN_ERR_INVALID_ARG, "text_softmax=%d must be 0 or 1", p->text_softmax);
  if (p->merge_mxfp8 != 0 && p->merge_mxfp8 != 1)
    return fail(VDN_ERR_INVALID_ARG, "merge_mxfp8=%d must be 0 or 1", p->merge_mxfp8);
  if (d->F % p->chunk_frames != 0)
    return fail(VDN_ERR_INVALID_ARG, "F=%d is not a multiple of chunk_frames=%d", d->F, p->chunk_frames);
  if (!(p->rms_eps >= 0.f) || !isfinite(p->text_init_scale) || !isfinite(p->softmax_scale))
    return fail(VDN_ERR_INVALID_ARG, "rms_eps / text_init_scale / softmax_scale not finite or negative eps");
  if (d->d_k != d->d_v) return fail(VDN_ERR_UNSUPPORTED, "d_k=%d != d_v=%d", d->d_k, d->d_v);
  if (d->d_k != 16 && d->d_k != 32 && d->d_k != 64 && d->d_k != 128)
    return fail(VDN_ERR_UNSUPPORTED, "head dim %d not in {16,32,64,128}", d->d_k);
  const long long L = (long long)d->F * d->N;
  const long long rows = (long long)d->B * d->H * L;
  if (L + d->T + 16 > (1ll << 31) - 1 || rows > (1ll << 40))
    return fail(VDN_ERR_INVALID_ARG, "sequence too long (L=%lld)", L);
  if (d->N > (1 << 26)) return fail(VDN_ERR_INVALID_ARG, "N=%d too large", d->N);
  g->B = d->B; g->H = d->H; g->F = d->F; g->N = d->N; g->T = d->T; g->D = d->d_k;
  g->cf = p->chunk_frames; g->wc = p->window_chunks; g->anchors = p->anchors;
  g->C = d->F / p->chunk_frames;
  g->L = L;
  g->Ts = p->text_softmax ? d->T : 0;
  return VDN_OK;
}

float softmax_scale(const vdn_params* p, int D) {
  return p->softmax_scale > 0.f ? p->softmax_scale : 1.f / sqrtf((float)D);
}

#define NEED(ptr) \
  if (!(ptr)) return fail(VDN_ERR_INVALID_ARG, "%s is NULL", #ptr)

// VDA stages a1-a4 into the workspace; P pointers may be workspace or caller buffers.
vdn_status run_scan(const vdn::Geometry& g, const vdn_params* p, vdn_dtype dt, const void* k,
                    const void* v, const float* beta, const float* alpha, const void* kt,
                    const void* vt, const float* bt, char* ws, const Layout& lay, float* P_fwd,
                    float* P_rev, hipStream_t s) {
  float* Tf = (float*)(ws + lay.Tf);
  float* Uf = (float*)(ws + lay.Uf);
  float* St = (float*)(ws + lay.St);
  float* Tc = (float*)(ws + lay.Tc);
  float* Uc = (float*)(ws + lay.Uc);
  if (dt == VDN_BF16)
    VDN_HIP(vdn::launch_vda_frame_solve<uint16_t>(g, (const uint16_t*)k, (const uint16_t*)v, beta,
                                                  alpha, (const uint16_t*)kt, (const uint16_t*)vt,
                                                  bt, Tf, Uf, St, s));
  else
    VDN_HIP(vdn::launch_vda_frame_solve<float>(g, (const float*)k, (const float*)v, beta, alpha,
                                               (const float*)kt, (const float*)vt, bt, Tf, Uf, St,
                                               s));
  // With all heads on one GPU the frame-level scan does fewer products than
  // composing chunks first and scanning those, and occupies far fewer
  // compute units (96 workgroups at H3 against ~4,600) beside the Softmax;
  // composition pays off once heads are sharded over GPUs.
  if (g.D == 64 || g.D == 128) {
    VDN_HIP(vdn::launch_vda_frame_scan(g, Tf, Uf, St, p->text_init_scale, P_fwd, P_rev, s));
    return VDN_OK;
  }
  const int dirs = (P_fwd ? 1 : 0) | (P_rev ? 2 : 0);
  VDN_HIP(vdn::launch_vda_chunk_compose(g, Tf, Uf, Tc, Uc, dirs, s));
  VDN_HIP(vdn::launch_vda_chunk_scan(g, Tc, Uc, St, p->text_init_scale, P_fwd, P_rev, s));
  return VDN_OK;
}

// The Softmax branch (a7).  With g.Ts > 0 the text keys k_text / v_text
// [B,H,Ts,d] are keys of every query as well.
vdn_status run_softmax(const vdn::Geometry& g, const vdn_params* p, vdn_dtype dt, const void* q,
                       const void* k, const void* v, const void* k_text, const void* v_text,
                       const float* g_s, void* out, float* lse, char* ws, const Layout& lay,
                       hipStream_t s) {
  const float sc = softmax_scale(p, g.D);
  const long long BH = (long long)g.B * g.H;
  if (dt == VDN_BF16 && vdn::window_softmax_mfma_ok(g)) {
    // V^T [B,H,D,Lp]: columns 0..L-1 the video values, then the text values
    // and zero padding up to Lp
    uint16_t* vt = (uint16_t*)(ws + lay.vt);
    const long long Lp = vdn::softmax_vt_pitch(g);
    VDN_HIP(vdn::launch_transpose_bf16((const uint16_t*)v, vt, g.L, g.L, g.D, Lp, Lp * g.D, BH, s));
    if (g.Ts > 0)
      VDN_HIP(vdn::launch_transpose_bf16((const uint16_t*)v_text, vt + g.L, Lp - g.L, g.Ts, g.D, Lp,
                                         Lp * g.D, BH, s));
    VDN_HIP(timer_mark(s, true));
    VDN_HIP(vdn::launch_window_softmax_mfma(g, (const uint16_t*)q, (const uint16_t*)k,
                                            (const uint16_t*)k_text, vt, g_s, (uint16_t*)out, lse,
                                            sc, s));
    VDN_HIP(timer_mark(s, false));
  } else if (dt == VDN_BF16) {
    VDN_HIP(timer_mark(s, true));
    VDN_HIP(vdn::launch_window_softmax_simt<uint16_t>(
        g, (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)k_text,
        (const uint16_t*)v_text, g_s, (uint16_t*)out, lse, sc, s));
    VDN_HIP(timer_mark(s, false));
  } else {
    VDN_HIP(timer_mark(s, true));
    VDN_HIP(vdn::launch_window_softmax_simt<float>(g, (const float*)q, (const float*)k,
                                                   (const float*)v, (const float*)k_text,
                                                   (const float*)v_text, g_s, (float*)out, lse,
                                                   sc, s));
    VDN_HIP(timer_mark(s, false));
  }
  return VDN_OK;
}

// Checks of the merge (a8) arguments shared by vdn_attn_fwd and vdn_merge_fwd.
vdn_status check_merge(const vdn::Geometry& g, const vdn_params* p, vdn_dtype dt, const void* W_s,
                       const void* W_l, int Dm) {
  if ((W_s == nullptr) != (W_l == nullptr))
    return fail(VDN_ERR_INVALID_ARG, "W_s and W_l must both be given or both be NULL");
  if (Dm < 1) return fail(VDN_ERR_INVALID_ARG, "D=%d must be >= 1", Dm);
  if (!W_s && Dm != g.H * g.D)
    return fail(VDN_ERR_INVALID_ARG, "without projections D=%d must equal H*d_v=%d", Dm, g.H * g.D);
  if (p->merge_mxfp8) {
    if (dt != VDN_BF16) return fail(VDN_ERR_UNSUPPORTED, "the MX-FP8 merge needs bf16 storage");
    if (!W_s) return fail(VDN_ERR_INVALID_ARG, "the MX-FP8 merge needs the projections W_s, W_l");
    if ((g.H * g.D) % 64 != 0 || Dm % 8 != 0)
      return fail(VDN_ERR_UNSUPPORTED, "the MX-FP8 merge needs H*d_v %% 64 == 0 and D %% 8 == 0");
  }
  return VDN_OK;
}

// Whether the layer's readout runs after the Softmax rather than beside it:
// when the Softmax's algorithmic work (4 d per visible query-key pair) is at
// least kReadoutAfterFlops.  Side by side on one MI355X the readout after
// the Softmax was 1% faster per layer step at 55 and 63 TFLOP of Softmax
// work and 3% slower at 2.2 TFLOP, where beside the Softmax it is nearly
// hidden.  Pairs from the window rule: a non-anchor query frame sees at most
// (2 wc + 1) cf frames plus the two anchors, an anchor frame every frame.
constexpr double kReadoutAfterFlops = 8e12;
bool readout_after_softmax(const vdn::Geometry& g) {
  const double win = std::min<double>(g.F, (2.0 * g.wc + 1) * g.cf + (g.anchors ? 2 : 0));
  const double qf = g.anchors ? std::max(g.F - 2, 0) : g.F;
  const double frame_pairs = qf * win + (g.anchors ? (double)std::min(g.F, 2) * g.F : 0.0);
  const double pairs = (double)g.B * g.H * (double)g.N * g.N * frame_pairs;
  return 4.0 * g.D * pairs >= kReadoutAfterFlops;
}

// Merge, part 1 (needs only the projections, so it may run on the linear
// branch's stream): transposed projections, and with MX-FP8 their operands.
vdn_status merge_prepare(const vdn::Geometry& g, const vdn_params* p, vdn_dtype dt, const void* W_s,
                         const void* W_l, int Dm, char* ws, const Layout& lay, hipStream_t s) {
  const int K = g.H * g.D;
  if (!W_s || dt != VDN_BF16) return VDN_OK;
  const bool mx = use_mx(p, dt);
  if (!mx && !(Dm % 8 == 0 && K % 64 == 0)) return VDN_OK;   // the SIMT GEMM reads W directly
  uint16_t* w0t = (uint16_t*)(ws + lay.wt0);
  uint16_t* w1t = (uint16_t*)(ws + lay.wt1);
  VDN_HIP(vdn::launch_transpose_bf16((const uint16_t*)W_s, w0t, K, K, Dm, K, (long long)K * Dm, 1, s));
  VDN_HIP(vdn::launch_transpose_bf16((const uint16_t*)W_l, w1t, K, K, Dm, K, (long long)K * Dm, 1, s));
  if (mx) {
    uint8_t* wc = (uint8_t*)(ws + lay.mxw);
    uint8_t* wsc = (uint8_t*)(ws + lay.mxws);
    VDN_HIP(vdn::launch_mx_quant_rows(w0t, Dm, K, wc, wsc, 2LL * K, 0, s));
    VDN_HIP(vdn::launch_mx_quant_rows(w1t, Dm, K, wc, wsc, 2LL * K, K, s));
  }
  return VDN_OK;
}

// Merge, part 2, on the caller's stream after both branches: out = [Ohat_s |
// Ohat_l] [W_s ; W_l] (or Ohat_s + Ohat_l without projections).
vdn_status merge_finish(const vdn::Geometry& g, const vdn_params* p, vdn_dtype dt, const void* W_s,
                        const void* W_l, const void* ohs, const void* ohl, void* out, int Dm,
                        char* ws, const Layout& lay, hipStream_t s) {
  const long long M = (long long)g.B * g.L;
  const int K = g.H * g.D;
  if (!W_s) {
    if (dt == VDN_BF16)
      VDN_HIP(vdn::launch_add<uint16_t>((const uint16_t*)ohs, (const uint16_t*)ohl, (uint16_t*)out,
                                        M * K, s));
    else
      VDN_HIP(vdn::launch_add<float>((const float*)ohs, (const float*)ohl, (float*)out, M * K, s));
  } else if (use_mx(p, dt)) {
    uint8_t* ac = (uint8_t*)(ws + lay.mxa);
    uint8_t* asc = (uint8_t*)(ws + lay.mxas);
    VDN_HIP(vdn::launch_mx_quant_rows((const uint16_t*)ohs, M, K, ac, asc, 2LL * K, 0, s));
    VDN_HIP(vdn::launch_mx_quant_rows((const uint16_t*)ohl, M, K, ac, asc, 2LL * K, K, s));
    VDN_HIP(vdn::launch_merge_gemm_mx(ac, asc, (const uint8_t*)(ws + lay.mxw),
                                      (const uint8_t*)(ws + lay.mxws), (uint16_t*)out, M, 2 * K,
                                      Dm, s));
  } else if (dt == VDN_BF16 && Dm % 8 == 0 && K % 64 == 0) {
    VDN_HIP(vdn::launch_merge_gemm_bf16((const uint16_t*)ohs, (const uint16_t*)ohl,
                                        (const uint16_t*)(ws + lay.wt0),
                                        (const uint16_t*)(ws + lay.wt1), (uint16_t*)out, M, K, Dm,
                                        s));
  } else if (dt == VDN_BF16) {
    VDN_HIP(vdn::launch_merge_gemm_simt<uint16_t>((const uint16_t*)ohs, (const uint16_t*)ohl,
                                                  (const uint16_t*)W_s, (const uint16_t*)W_l,
                                                  (uint16_t*)out, M, K, Dm, s));
  } else {
    VDN_HIP(vdn::launch_merge_gemm_simt<float>((const float*)ohs, (const float*)ohl,
                                               (const float*)W_s, (const float*)W_l, (float*)out,
                                               M, K, Dm, s));
  }
  return VDN_OK;
}

// Scratch of the allocation-free Softmax entry point: a file-scope device
// array (each GPU the library runs on holds its own copy until the process
// ends).  In host code `scratch` names a host-side stand-in, so its device
// address is looked up once per device (with that device current) and kept.
constexpr size_t kNoAllocScratchBytes = 64ull << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

struct ScratchAddr {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchAddr g_scratch[16];

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 16) return hipErrorInvalidDevice;
  ScratchAddr& sa = g_scratch[dev];
  std::call_once(sa.once, [&sa] { sa.err = hipGetSymbolAddress(&sa.ptr, HIP_SYMBOL(scratch)); });
  if (sa.err != hipSuccess) return sa.err;
  *out = sa.ptr;
  return hipSuccess;
}

vdn_status check_workspace(void* ws, size_t bytes, size_t need) {
  if (bytes < need)
    return fail(VDN_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", bytes, need);
  if (need && !ws) return fail(VDN_ERR_INVALID_ARG, "workspace is NULL");
  if ((uintptr_t)ws & 255) return fail(VDN_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  return VDN_OK;
}

vdn_status scan_entry(const void* k, const void* v, const float* beta, const float* alpha,
                      const void* k_text, const void* v_text, const float* beta_text, float* P_fwd,
                      float* P_rev, float* S_text_out, void* workspace, size_t workspace_bytes,
                      const vdn_dims* dims, const vdn_params* p, vdn_dtype dt, void* stream) {
  g_err[0] = 0;
  vdn::Geometry g;
  vdn_status st = check_geometry(dims, p, dt, &g);
  if (st != VDN_OK) return st;
  NEED(k); NEED(v); NEED(beta); NEED(alpha);
  if (g.T > 0) { NEED(k_text); NEED(v_text); NEED(beta_text); }
  if (!P_fwd && !P_rev) return fail(VDN_ERR_INVALID_ARG, "output state pointer is NULL");
  const Layout lay = make_layout(g, g.H * g.D, dt, false, Entry::Scan);
  st = check_workspace(workspace, workspace_bytes, lay.total);
  if (st != VDN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  st = run_scan(g, p, dt, k, v, beta, alpha, k_text, v_text, beta_text, ws, lay, P_fwd, P_rev, s);
  if (st != VDN_OK) return st;
  if (S_text_out)
    VDN_HIP(hipMemcpyAsync(S_text_out, ws + lay.St, (size_t)g.B * g.H * g.D * g.D * 4,
                           hipMemcpyDeviceToDevice, s));
  return VDN_OK;
}

}  // namespace

extern "C" {

void vdn_default_params(vdn_params* p) {
  if (p) *p = defaults();
}

const char* vdn_status_string(vdn_status s) {
  switch (s) {
    case VDN_OK: return "VDN_OK";
    case VDN_ERR_INVALID_ARG: return "VDN_ERR_INVALID_ARG";
    case VDN_ERR_UNSUPPORTED: return "VDN_ERR_UNSUPPORTED";
    case VDN_ERR_WORKSPACE: return "VDN_ERR_WORKSPACE";
    case VDN_ERR_HIP: return "VDN_ERR_HIP";
    default: break;
  }
  return "unknown vdn_status";
}

const char* vdn_last_error(void) { return g_err; }

void vdn_timer_disable(void) {
  if (g_timer.ev) {
    for (int i = 0; i < 2 * g_timer.cap; ++i) (void)hipEventDestroy(g_timer.ev[i]);
    delete[] g_timer.ev;
  }
  g_timer = KernelTimer{};
}

vdn_status vdn_timer_enable(int n) {
  g_err[0] = 0;
  vdn_timer_disable();
  if (n < 1 || n > (1 << 20)) return fail(VDN_ERR_INVALID_ARG, "timer capacity %d out of range", n);
  g_timer.ev = new hipEvent_t[2 * (size_t)n];
  for (int i = 0; i < 2 * n; ++i) {
    hipError_t e = hipEventCreate(&g_timer.ev[i]);
    if (e != hipSuccess) {
      g_timer.cap = i / 2;   // destroy what was created
      for (int j = i; j < 2 * n; ++j) g_timer.ev[j] = nullptr;
      for (int j = 0; j < i; ++j) (void)hipEventDestroy(g_timer.ev[j]);
      delete[] g_timer.ev;
      g_timer = KernelTimer{};
      return fail(VDN_ERR_HIP, "hipEventCreate failed: %s", hipGetErrorString(e));
    }
  }
  g_timer.cap = n;
  g_timer.used = 0;
  return VDN_OK;
}

int vdn_timer_read(float* ms, int cap) {
  g_err[0] = 0;
  if (!ms) return fail(VDN_ERR_INVALID_ARG, "ms is NULL");
  const int n = g_timer.used < cap ? g_timer.used : cap;
  for (int i = 0; i < n; ++i) {
    hipError_t e = hipEventSynchronize(g_timer.ev[2 * i + 1]);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms[i], g_timer.ev[2 * i], g_timer.ev[2 * i + 1]);
    if (e != hipSuccess) return fail(VDN_ERR_HIP, "timer read failed: %s", hipGetErrorString(e));
  }
  return n;
}

size_t vdn_workspace_bytes(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt) {
  vdn::Geometry g;
  if (check_geometry(dims, p, dt, &g) != VDN_OK) return 0;
  const int Dm = dims->D > 0 ? dims->D : g.H * g.D;
  return make_layout(g, Dm, dt, use_mx(p, dt), Entry::Attn).total;
}

size_t vdn_scan_workspace_bytes(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt) {
  vdn::Geometry g;
  if (check_geometry(dims, p, dt, &g) != VDN_OK) return 0;
  return make_layout(g, g.H * g.D, dt, false, Entry::Scan).total;
}

size_t vdn_softmax_workspace_bytes(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt) {
  vdn::Geometry g;
  if (check_geometry(dims, p, dt, &g) != VDN_OK) return 0;
  return make_layout(g, g.H * g.D, dt, false, Entry::Softmax).total;
}

size_t vdn_merge_workspace_bytes(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt) {
  vdn::Geometry g;
  if (check_geometry(dims, p, dt, &g) != VDN_OK || dims->D < 1) return 0;
  return make_layout(g, dims->D, dt, use_mx(p, dt), Entry::Merge).total;
}

vdn_status vdn_window_plan(int F, const vdn_params* p, uint8_t* vis, int32_t* i_fwd, int32_t* ws,
                           int32_t* i_rev, int32_t* we) {
  g_err[0] = 0;
  if (!p) return fail(VDN_ERR_INVALID_ARG, "params is NULL");
  if (F < 2) return fail(VDN_ERR_INVALID_ARG, "F=%d must be >= 2", F);
  if (p->chunk_frames < 1 || p->window_chunks < 0 || (p->anchors != 0 && p->anchors != 1))
    return fail(VDN_ERR_INVALID_ARG, "bad chunk_frames/window_chunks/anchors");
  if (F % p->chunk_frames != 0)
    return fail(VDN_ERR_INVALID_ARG, "F=%d is not a multiple of chunk_frames=%d", F, p->chunk_frames);
  // One head with one token per frame: the Softmax kernels' own item decoder
  // run over their whole grid gives every query frame's key frames.
  vdn::Geometry g{};
  g.B = 1; g.H = 1; g.F = F; g.N = 1; g.T = 0; g.D = 0;
  g.cf = p->chunk_frames; g.wc = p->window_chunks; g.anchors = p->anchors;
  g.C = F / g.cf; g.L = F; g.Ts = 0;
  if (vis) {
    memset(vis, 0, (size_t)F * F);
    const vdn::SoftmaxWork w = vdn::window_work(g, vdn::kWinMfmaBQ);
    int* covered = new int[F]();
    for (int bid = 0; bid < w.grid; ++bid) {
      vdn::Item it;
      int q0;
      if (!vdn::decode_item<false>(g, w, vdn::kWinMfmaBQ, bid, 0, it, q0)) continue;
      const int q1 = q0 + vdn::kWinMfmaBQ < it.q_end ? q0 + vdn::kWinMfmaBQ : it.q_end;
      const int kb[3] = {it.kb0, it.kb1, it.kb2}, ke[3] = {it.ke0, it.ke1, it.ke2};
      for (int t = q0; t < q1; ++t) {
        ++covered[t];
        for (int s = 0; s < it.nspan; ++s)
          for (int f = kb[s]; f < ke[s]; ++f) vis[(size_t)t * F + f] = 1;
      }
    }
    int bad = -1;
    for (int t = 0; t < F && bad < 0; ++t)
      if (covered[t] != 1) bad = t;
    const int nbad = bad >= 0 ? covered[bad] : 0;
    delete[] covered;
    if (bad >= 0)
      return fail(VDN_ERR_UNSUPPORTED, "work items cover query frame %d %d times", bad, nbad);
  }
  // gather indices and bridge ends: the readout kernels' own function
  for (int t = 0; t < F; ++t) {
    int a, s, b, e;
    vdn::readout_indices(g, t, a, s, b, e);
    if (i_fwd) i_fwd[t] = a;
    if (ws) ws[t] = s;
    if (i_rev) i_rev[t] = b;
    if (we) we[t] = e;
  }
  return VDN_OK;
}

vdn_status vdn_window_row_keys(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt,
                               int64_t* keys) {
  g_err[0] = 0;
  vdn::Geometry g;
  vdn_status st = check_geometry(dims, p, dt, &g);
  if (st != VDN_OK) return st;
  NEED(keys);
  const long long rows = (long long)g.B * g.H * g.L;
  if (rows > (1ll << 31)) return fail(VDN_ERR_INVALID_ARG, "too many rows (%lld)", rows);
  // the launch vdn_window_softmax_fwd makes for these sizes
  const bool mfma = dt == VDN_BF16 && vdn::window_softmax_mfma_ok(g);
  const int bq = mfma ? vdn::kWinMfmaBQ : vdn::kWinSimtBQ;
  // the MFMA kernel walks the text keys in whole 16-key groups and takes
  // the last Ts % 16 as one masked block after the walk
  const int nt = mfma ? (g.Ts & ~15) : g.Ts;
  const int rem = g.Ts - nt;
  const vdn::SoftmaxWork w = vdn::window_work(g, bq);
  int* covered = new int[rows]();
  memset(keys, 0, (size_t)rows * sizeof(int64_t));
  for (int bid = 0; bid < w.grid; ++bid) {
    vdn::Item it;
    int q0;
    if (!vdn::decode_item<true>(g, w, bq, bid, nt, it, q0)) continue;
    const int kb[4] = {it.kb0, it.kb1, it.kb2, it.kb3}, ke[4] = {it.ke0, it.ke1, it.ke2, it.ke3};
    long long n = rem;
    for (int s = 0; s < it.nspan; ++s) n += ke[s] - kb[s];
    const int q1 = q0 + bq < it.q_end ? q0 + bq : it.q_end;
    for (int l = q0; l < q1; ++l) {
      const long long r = (long long)it.bh * g.L + l;
      ++covered[r];
      keys[r] += n;
    }
  }
  for (long long r = 0; r < rows; ++r)
    if (covered[r] != 1) keys[r] = -1;
  delete[] covered;
  return VDN_OK;
}

vdn_status vda_scan_fwd(const void* k, const void* v, const float* beta, const float* alpha,
                        const void* k_text, const void* v_text, const float* beta_text,
                        float* P_fwd, float* S_text_out, void* workspace, size_t workspace_bytes,
                        const vdn_dims* dims, const vdn_params* p, vdn_dtype dt, void* stream) {
  if (!P_fwd) { g_err[0] = 0; return fail(VDN_ERR_INVALID_ARG, "P_fwd is NULL"); }
  return scan_entry(k, v, beta, alpha, k_text, v_text, beta_text, P_fwd, nullptr, S_text_out,
                    workspace, workspace_bytes, dims, p, dt, stream);
}

vdn_status vda_scan_rev(const void* k, const void* v, const float* beta, const float* alpha,
                        const void* k_text, const void* v_text, const float* beta_text,
                        float* P_rev, float* S_text_out, void* workspace, size_t workspace_bytes,
                        const vdn_dims* dims, const vdn_params* p, vdn_dtype dt, void* stream) {
  if (!P_rev) { g_err[0] = 0; return fail(VDN_ERR_INVALID_ARG, "P_rev is NULL"); }
  return scan_entry(k, v, beta, alpha, k_text, v_text, beta_text, nullptr, P_rev, S_text_out,
                    workspace, workspace_bytes, dims, p, dt, stream);
}

vdn_status vdn_window_softmax_fwd(const void* q, const void* k, const void* v,
                                  const void* k_text, const void* v_text, const float* g_s,
                                  void* out, float* lse, void* workspace, size_t workspace_bytes,
                                  const vdn_dims* dims, const vdn_params* p, vdn_dtype dt,
                                  void* stream) {
  g_err[0] = 0;
  vdn::Geometry g;
  vdn_status st = check_geometry(dims, p, dt, &g);
  if (st != VDN_OK) return st;
  NEED(q); NEED(k); NEED(v); NEED(out);
  if (g.Ts > 0) { NEED(k_text); NEED(v_text); }
  const Layout lay = make_layout(g, g.H * g.D, dt, false, Entry::Softmax);
  st = check_workspace(workspace, workspace_bytes, lay.total);
  if (st != VDN_OK) return st;
  return run_softmax(g, p, dt, q, k, v, k_text, v_text, g_s, out, lse, (char*)workspace, lay,
                     (hipStream_t)stream);
}

vdn_status vdn_window_softmax_fwd_noalloc(const void* q, const void* k, const void* v,
                                          const void* k_text, const void* v_text, const float* g_s,
                                          void* out, float* lse, const vdn_dims* dims,
                                          const vdn_params* p, vdn_dtype dt, void* stream) {
  g_err[0] = 0;
  vdn::Geometry g;
  vdn_status st = check_geometry(dims, p, dt, &g);
  if (st != VDN_OK) return st;
  NEED(q); NEED(k); NEED(v); NEED(out);
  if (g.Ts > 0) { NEED(k_text); NEED(v_text); }
  // the same regions vdn_window_softmax_fwd takes from its workspace (V^T
  // and the text values, every element rewritten by each call), here in the
  // device array
  const Layout lay = make_layout(g, g.H * g.D, dt, false, Entry::Softmax);
  if (lay.total > kNoAllocScratchBytes)
    return fail(VDN_ERR_UNSUPPORTED,
                "vdn_window_softmax_fwd_noalloc: these sizes need %zu bytes of scratch, more than "
                "its %zu-byte device array; use vdn_window_softmax_fwd with a workspace",
                lay.total, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (lay.total > 0) VDN_HIP(scratch_address(&ws));
  return run_softmax(g, p, dt, q, k, v, k_text, v_text, g_s, out, lse, (char*)ws, lay,
                     (hipStream_t)stream);
}

vdn_status vdn_attn_fwd(const void* q, const void* k, const void* v, const float* beta,
                        const float* alpha, const void* k_text, const void* v_text,
                        const float* beta_text, const float* g_s, const float* g_l,
                        const float* gamma, const void* W_s, const void* W_l, void* out,
                        void* ohat_s, void* ohat_l, void* workspace, size_t workspace_bytes,
                        const vdn_dims* dims, const vdn_params* p, vdn_dtype dt, void* stream) {
  g_err[0] = 0;
  vdn::Geometry g;
  vdn_status st = check_geometry(dims, p, dt, &g);
  if (st != VDN_OK) return st;
  NEED(q); NEED(k); NEED(v); NEED(beta); NEED(alpha); NEED(g_s); NEED(g_l); NEED(out);
  if (g.T > 0) { NEED(k_text); NEED(v_text); NEED(beta_text); }
  const int Dm = dims->D;
  st = check_merge(g, p, dt, W_s, W_l, Dm);
  if (st != VDN_OK) return st;
  const Layout lay = make_layout(g, Dm, dt, use_mx(p, dt), Entry::Attn);
  // the branch-output regions come last: not needed when the caller passes both
  st = check_workspace(workspace, workspace_bytes, ohat_s && ohat_l ? lay.ohs : lay.total);
  if (st != VDN_OK) return st;

  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  void* ohs = ohat_s ? ohat_s : (void*)(ws + lay.ohs);
  void* ohl = ohat_l ? ohat_l : (void*)(ws + lay.ohl);
  float* Pf = (float*)(ws + lay.Pf);
  float* Pr = (float*)(ws + lay.Pr);

  // The linear branch (a1-a6) on the side stream, forked from and joined
  // back into the caller's stream; the window Softmax (a7) runs on the
  // caller's stream meanwhile.  The two touch disjoint workspace regions.
  // Beside a long Softmax each readout (a5, a6) workgroup waits for a whole
  // compute unit and then holds it for a stretched span, which costs the
  // Softmax about twice the readout's own time; there the readout follows
  // the Softmax on the caller's stream instead.
  const bool ro_after = readout_after_softmax(g);
  auto readout = [&](hipStream_t rs) -> vdn_status {
    const hipError_t e = dt == VDN_BF16
        ? vdn::launch_vda_readout<uint16_t>(g, (const uint16_t*)q, alpha, Pf, Pr, g_l, gamma,
                                            p->rms_eps, (uint16_t*)ohl, rs)
        : vdn::launch_vda_readout<float>(g, (const float*)q, alpha, Pf, Pr, g_l, gamma,
                                         p->rms_eps, (float*)ohl, rs);
    return e == hipSuccess ? VDN_OK : fail(VDN_ERR_HIP, "readout launch failed: %s", hipGetErrorString(e));
  };
  SideStream* ss = nullptr;
  VDN_HIP(side_stream(&ss));
  VDN_HIP(hipEventRecord(ss->fork, s));
  VDN_HIP(hipStreamWaitEvent(ss->stream, ss->fork, 0));
  st = run_scan(g, p, dt, k, v, beta, alpha, k_text, v_text, beta_text, ws, lay, Pf, Pr, ss->stream);
  if (st == VDN_OK && !ro_after) st = readout(ss->stream);
  // the merge's projection transposes (and MX-FP8 operands of W) also run
  // on the side stream, off the Softmax's path
  if (st == VDN_OK) st = merge_prepare(g, p, dt, W_s, W_l, Dm, ws, lay, ss->stream);
  // join is recorded even after a failure, so the caller's stream never
  // runs ahead of work already queued on the side stream
  const hipError_t ej = hipEventRecord(ss->join, ss->stream);
  if (st == VDN_OK)
    st = run_softmax(g, p, dt, q, k, v, k_text, v_text, g_s, ohs, nullptr, ws, lay, s);
  const hipError_t ew = ej == hipSuccess ? hipStreamWaitEvent(s, ss->join, 0) : ej;
  if (st != VDN_OK) return st;
  if (ew != hipSuccess) return fail(VDN_ERR_HIP, "side-stream join failed: %s", hipGetErrorString(ew));
  if (ro_after) {
    st = readout(s);
    if (st != VDN_OK) return st;
  }
  // Merge (a8)
  return merge_finish(g, p, dt, W_s, W_l, ohs, ohl, out, Dm, ws, lay, s);
}

vdn_status vdn_merge_fwd(const void* ohat_s, const void* ohat_l, const void* W_s, const void* W_l,
                         void* out, void* workspace, size_t workspace_bytes, const vdn_dims* dims,
                         const vdn_params* p, vdn_dtype dt, void* stream) {
  g_err[0] = 0;
  vdn::Geometry g;
  vdn_status st = check_geometry(dims, p, dt, &g);
  if (st != VDN_OK) return st;
  NEED(ohat_s); NEED(ohat_l); NEED(out);
  const int Dm = dims->D;
  st = check_merge(g, p, dt, W_s, W_l, Dm);
  if (st != VDN_OK) return st;
  const Layout lay = make_layout(g, Dm, dt, use_mx(p, dt), Entry::Merge);
  st = check_workspace(workspace, workspace_bytes, lay.total);
  if (st != VDN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  st = merge_prepare(g, p, dt, W_s, W_l, Dm, ws, lay, s);
  if (st != VDN_OK) return st;
  return merge_finish(g, p, dt, W_s, W_l, ohat_s, ohat_l, out, Dm, ws, lay, s);
}

// Merge backward: dOhat = dout W^T on the merge's GEMM; dW = Ohat^T dout
// over the tokens, from transposed copies of dout and of each Ohat.
struct MergeBwdLayout {
  size_t doutT, ohT, total;
};

MergeBwdLayout merge_bwd_layout(const vdn::Geometry& g, int Dm) {
  const size_t M = (size_t)g.B * g.L, K = (size_t)g.H * g.D;
  MergeBwdLayout l{};
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t r = o; o += align256(bytes); return r; };
  l.doutT = take(M * Dm * 2);
  l.ohT = take(M * K * 2);
  l.total = o;
  return l;
}

size_t vdn_merge_bwd_workspace_bytes(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt) {
  vdn::Geometry g;
  if (check_geometry(dims, p, dt, &g) != VDN_OK || dims->D < 1) return 0;
  return merge_bwd_layout(g, dims->D).total;
}

vdn_status vdn_merge_bwd(const void* ohat_s, const void* ohat_l, const void* W_s, const void* W_l,
                         const void* d_out, void* d_ohat_s, void* d_ohat_l, void* dW_s, void* dW_l,
                         void* workspace, size_t workspace_bytes, const vdn_dims* dims,
                         const vdn_params* p, vdn_dtype dt, void* stream) {
  g_err[0] = 0;
  vdn::Geometry g;
  vdn_status st = check_geometry(dims, p, dt, &g);
  if (st != VDN_OK) return st;
  NEED(d_out); NEED(d_ohat_s); NEED(d_ohat_l);
  const int Dm = dims->D;
  if ((W_s == nullptr) != (W_l == nullptr))
    return fail(VDN_ERR_INVALID_ARG, "W_s and W_l must both be given or both be NULL");
  if ((dW_s == nullptr) != (dW_l == nullptr))
    return fail(VDN_ERR_INVALID_ARG, "dW_s and dW_l must both be given or both be NULL");
  const long long M = (long long)g.B * g.L;
  const int K = g.H * g.D;
  hipStream_t s = (hipStream_t)stream;
  const size_t es = dt == VDN_BF16 ? 2 : 4;
  if (!W_s) {   // out = Ohat_s + Ohat_l
    if (Dm != K) return fail(VDN_ERR_INVALID_ARG, "without projections D=%d must equal H*d_v=%d", Dm, K);
    if (dW_s) return fail(VDN_ERR_INVALID_ARG, "no projections: dW_s, dW_l must be NULL");
    VDN_HIP(hipMemcpyAsync(d_ohat_s, d_out, (size_t)M * K * es, hipMemcpyDeviceToDevice, s));
    VDN_HIP(hipMemcpyAsync(d_ohat_l, d_out, (size_t)M * K * es, hipMemcpyDeviceToDevice, s));
    return VDN_OK;
  }
  if (dt != VDN_BF16) return fail(VDN_ERR_UNSUPPORTED, "the merge backward needs bf16 storage");
  if (Dm % 128 != 0 || K % 8 != 0)
    return fail(VDN_ERR_UNSUPPORTED, "the merge backward needs D %% 128 == 0 and H*d_v %% 8 == 0");
  if ((long long)M * Dm * 2 > 0x7FFFFFF0ll || (long long)M * K * 2 > 0x7FFFFFF0ll)
    return fail(VDN_ERR_UNSUPPORTED, "the merge backward's operands must stay below 2 GiB");
  if (dW_s) {
    NEED(ohat_s); NEED(ohat_l);
    if (M % 128 != 0) return fail(VDN_ERR_UNSUPPORTED, "dW needs B*L %% 128 == 0 (B*L=%lld)", M);
  }
  const MergeBwdLayout lay = merge_bwd_layout(g, Dm);
  if (dW_s) {
    st = check_workspace(workspace, workspace_bytes, lay.total);
    if (st != VDN_OK) return st;
  }
  // dW_* [K, D] = Ohat_*^T dout, on the side stream: both operands transposed
  // to token-contiguous rows.  Its GEMMs have few output tiles (K/256 x D/256)
  // and a long contraction, so they leave compute units free for the dOhat
  // GEMMs on the caller's stream.
  SideStream* ss = nullptr;
  hipError_t ej = hipSuccess;
  if (dW_s) {
    VDN_HIP(side_stream(&ss));
    VDN_HIP(hipEventRecord(ss->fork, s));
    VDN_HIP(hipStreamWaitEvent(ss->stream, ss->fork, 0));
    char* ws = (char*)workspace;
    uint16_t* doutT = (uint16_t*)(ws + lay.doutT);
    uint16_t* ohT = (uint16_t*)(ws + lay.ohT);
    hipError_t e = vdn::launch_transpose_bf16((const uint16_t*)d_out, doutT, M, M, Dm, M, M * Dm, 1,
                                              ss->stream);
    const void* oh[2] = {ohat_s, ohat_l};
    void* dw[2] = {dW_s, dW_l};
    for (int i = 0; i < 2 && e == hipSuccess; ++i) {
      e = vdn::launch_transpose_bf16((const uint16_t*)oh[i], ohT, M, M, K, M, M * K, 1, ss->stream);
      if (e == hipSuccess) e = vdn::launch_gemm_nt_bf16(ohT, doutT, (uint16_t*)dw[i], K, M, Dm, ss->stream);
    }
    // the join is recorded even after a failure, so the caller's stream
    // never runs ahead of work already queued on the side stream
    ej = hipEventRecord(ss->join, ss->stream);
    if (e != hipSuccess) st = fail(VDN_ERR_HIP, "weight-gradient launch failed: %s", hipGetErrorString(e));
  }
  // dOhat_* [M, K] = dout [M, D] W_*^T (W_* [K, D] is the contraction-contiguous right operand)
  hipError_t e2 = hipSuccess;
  if (st == VDN_OK) {
    e2 = vdn::launch_gemm_nt_bf16((const uint16_t*)d_out, (const uint16_t*)W_s, (uint16_t*)d_ohat_s, M,
                                  Dm, K, s);
    if (e2 == hipSuccess)
      e2 = vdn::launch_gemm_nt_bf16((const uint16_t*)d_out, (const uint16_t*)W_l, (uint16_t*)d_ohat_l,
                                    M, Dm, K, s);
  }
  const hipError_t ew = ss ? (ej == hipSuccess ? hipStreamWaitEvent(s, ss->join, 0) : ej) : hipSuccess;
  if (st != VDN_OK) return st;
  if (e2 != hipSuccess) return fail(VDN_ERR_HIP, "GEMM launch failed: %s", hipGetErrorString(e2));
  if (ew != hipSuccess) return fail(VDN_ERR_HIP, "side-stream join failed: %s", hipGetErrorString(ew));
  return VDN_OK;
}

size_t vdn_softmax_bwd_workspace_bytes(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt) {
  vdn::Geometry g;
  if (check_geometry(dims, p, dt, &g) != VDN_OK) return 0;
  return bwd_layout(g, dt).total;
}

vdn_status vdn_window_softmax_bwd(const void* q, const void* k, const void* v, const void* k_text,
                                  const void* v_text, const void* o, const float* lse,
                                  const float* g_s, const void* d_out, void* dq, void* dk, void* dv,
                                  void* dk_text, void* dv_text, float* dg_s, void* workspace,
                                  size_t workspace_bytes, const vdn_dims* dims, const vdn_params* p,
                                  vdn_dtype dt, void* stream) {
  g_err[0] = 0;
  vdn::Geometry g;
  vdn_status st = check_geometry(dims, p, dt, &g);
  if (st != VDN_OK) return st;
  NEED(q); NEED(k); NEED(v); NEED(o); NEED(lse); NEED(d_out); NEED(dq); NEED(dk); NEED(dv);
  if (g.Ts > 0) { NEED(k_text); NEED(v_text); NEED(dk_text); NEED(dv_text); }
  const BwdLayout lay = bwd_layout(g, dt);
  st = check_workspace(workspace, workspace_bytes, lay.total);
  if (st != VDN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  float* Dq = (float*)(ws + lay.Dq);
  const float sc = softmax_scale(p, g.D);
  vdn::SoftmaxBwdText tx;
  if (g.Ts > 0) {
    tx.k_text = k_text; tx.v_text = v_text; tx.dk_text = dk_text; tx.dv_text = dv_text;
  }
  if (dt == VDN_BF16) {
    uint16_t* dohm = (uint16_t*)(ws + lay.dohm);
    VDN_HIP(vdn::launch_softmax_bwd_prep<uint16_t>(g, (const uint16_t*)o, (const uint16_t*)d_out, g_s,
                                                   dohm, Dq, dg_s, s));
    if (vdn::softmax_bwd_mfma_ok(g)) {
      VDN_HIP(timer_mark(s, true));
      VDN_HIP(vdn::launch_softmax_bwd_mfma(g, (const uint16_t*)q, (const uint16_t*)k,
                                           (const uint16_t*)v, dohm, lse, Dq,
                                           (uint16_t*)dq, (uint16_t*)dk, (uint16_t*)dv, tx, sc, s));
      VDN_HIP(timer_mark(s, false));
    } else {
      VDN_HIP(vdn::launch_softmax_bwd_simt<uint16_t>(g, (const uint16_t*)q, (const uint16_t*)k,
                                                     (const uint16_t*)v, dohm, lse, Dq,
                                                     (uint16_t*)dq, (uint16_t*)dk, (uint16_t*)dv,
                                                     tx, sc, s));
    }
  } else {
    float* dohm = (float*)(ws + lay.dohm);
    VDN_HIP(vdn::launch_softmax_bwd_prep<float>(g, (const float*)o, (const float*)d_out, g_s, dohm,
                                                Dq, dg_s, s));
    VDN_HIP(vdn::launch_softmax_bwd_simt<float>(g, (const float*)q, (const float*)k, (const float*)v,
                                                dohm, lse, Dq, (float*)dq, (float*)dk, (float*)dv,
                                                tx, sc, s));
  }
  return VDN_OK;
}

size_t vda_bwd_workspace_bytes(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt) {
  vdn::Geometry g;
  if (check_geometry(dims, p, dt, &g) != VDN_OK) return 0;
  return vda_bwd_layout(g).total;
}

vdn_status vda_bwd(const void* q, const void* k, const void* v, const float* beta,
                   const float* alpha, const void* k_text, const void* v_text,
                   const float* beta_text, const float* g_l, const float* gamma, const void* d_out,
                   void* dq, void* dk, void* dv, float* dbeta, float* dalpha, void* dk_text,
                   void* dv_text, float* dbeta_text, float* dg_l, float* dgamma, void* workspace,
                   size_t workspace_bytes, const vdn_dims* dims, const vdn_params* p, vdn_dtype dt,
                   void* stream) {
  g_err[0] = 0;
  vdn::Geometry g;
  vdn_status st = check_geometry(dims, p, dt, &g);
  if (st != VDN_OK) return st;
  NEED(q); NEED(k); NEED(v); NEED(beta); NEED(alpha); NEED(g_l); NEED(d_out);
  NEED(dq); NEED(dk); NEED(dv); NEED(dbeta); NEED(dalpha);
  if (g.T > 0) {
    NEED(k_text); NEED(v_text); NEED(beta_text); NEED(dk_text); NEED(dv_text); NEED(dbeta_text);
  }
  if (g.F > 1024) return fail(VDN_ERR_UNSUPPORTED, "F=%d: the linear-branch backward supports F <= 1024", g.F);
  const VdaBwdLayout lay = vda_bwd_layout(g);
  st = check_workspace(workspace, workspace_bytes, lay.total);
  if (st != VDN_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  auto fp = [&](size_t off) { return (float*)(ws + off); };
  // forward recompute: frame maps and inverses, chunk maps, boundary states
  if (dt == VDN_BF16)
    VDN_HIP(vdn::launch_vda_frame_solve<uint16_t>(g, (const uint16_t*)k, (const uint16_t*)v, beta, alpha,
                                                  (const uint16_t*)k_text, (const uint16_t*)v_text,
                                                  beta_text, fp(lay.Tf), fp(lay.Uf), fp(lay.St), s,
                                                  fp(lay.Xf)));
  else
    VDN_HIP(vdn::launch_vda_frame_solve<float>(g, (const float*)k, (const float*)v, beta, alpha,
                                               (const float*)k_text, (const float*)v_text, beta_text,
                                               fp(lay.Tf), fp(lay.Uf), fp(lay.St), s, fp(lay.Xf)));
  VDN_HIP(vdn::launch_vda_chunk_compose(g, fp(lay.Tf), fp(lay.Uf), fp(lay.Tc), fp(lay.Uc), 3, s));
  VDN_HIP(vdn::launch_vda_chunk_scan(g, fp(lay.Tc), fp(lay.Uc), fp(lay.St), p->text_init_scale,
                                     fp(lay.Pf), fp(lay.Pr), s));
  vdn::VdaBwdPtrs bp{beta, alpha, beta_text, g_l, gamma,
                     fp(lay.Tf), fp(lay.Uf), fp(lay.Pf), fp(lay.Pr), fp(lay.St), fp(lay.Xf), fp(lay.Tc),
                     fp(lay.G), fp(lay.Dbr), fp(lay.dDbr), fp(lay.dgp), fp(lay.dP), fp(lay.mu),
                     fp(lay.Sst), fp(lay.Zst), fp(lay.ZT), fp(lay.Rscr),
                     dbeta, dalpha, dbeta_text, dg_l, dgamma};
  // the kernel timer (when enabled) brackets the readout adjoint, the longest kernel
  for (int stage = 0; stage < 2; ++stage) {
    if (stage == 0) VDN_HIP(timer_mark(s, true));
    if (dt == VDN_BF16)
      VDN_HIP(vdn::launch_vda_bwd<uint16_t>(g, bp, (const uint16_t*)q, (const uint16_t*)k,
                                            (const uint16_t*)v, (const uint16_t*)k_text,
                                            (const uint16_t*)v_text, (const uint16_t*)d_out,
                                            (uint16_t*)dq, (uint16_t*)dk, (uint16_t*)dv,
                                            (uint16_t*)dk_text, (uint16_t*)dv_text, p->rms_eps,
                                            p->text_init_scale, stage, s));
    else
      VDN_HIP(vdn::launch_vda_bwd<float>(g, bp, (const float*)q, (const float*)k, (const float*)v,
                                         (const float*)k_text, (const float*)v_text,
                                         (const float*)d_out, (float*)dq, (float*)dk, (float*)dv,
                                         (float*)dk_text, (float*)dv_text, p->rms_eps,
                                         p->text_init_scale, stage, s));
    if (stage == 0) VDN_HIP(timer_mark(s, false));
  }
  return VDN_OK;
}

vdn_status vdn_mx_quantize(const void* src, void* codes, void* scales, long long rows, int cols,
                           void* stream) {
  g_err[0] = 0;
  NEED(src); NEED(codes); NEED(scales);
  if (rows < 0 || cols < 0) return fail(VDN_ERR_INVALID_ARG, "rows=%lld cols=%d", rows, cols);
  if (cols % 32) return fail(VDN_ERR_INVALID_ARG, "cols=%d is not a multiple of 32", cols);
  if (rows * (long long)(cols / 32) > (1ll << 40)) return fail(VDN_ERR_INVALID_ARG, "too many blocks");
  VDN_HIP(vdn::launch_mx_quant_rows((const uint16_t*)src, rows, cols, (uint8_t*)codes,
                                    (uint8_t*)scales, cols, 0, (hipStream_t)stream));
  return VDN_OK;
}

void vda_prep_default_params(vda_prep_params* p, int grid_h, int grid_w) {
  if (!p) return;
  p->grid_h = grid_h;
  p->grid_w = grid_w;
  p->kernel_h = 3;
  p->kernel_w = 3;
  p->taps = 5;
  p->causal = 0;
  p->l2_eps = 1e-6f;
}

vdn_status vda_prep_fwd(const void* q, const void* k, const void* v, const float* w_spatial,
                        const float* w_temporal, void* q_out, void* k_out, void* v_out,
                        const vdn_dims* dims, const vda_prep_params* p, vdn_dtype dt,
                        void* stream) {
  g_err[0] = 0;
  if (!dims) return fail(VDN_ERR_INVALID_ARG, "dims is NULL");
  if (!p) return fail(VDN_ERR_INVALID_ARG, "params is NULL");
  NEED(q); NEED(k); NEED(v); NEED(w_spatial); NEED(w_temporal);
  NEED(q_out); NEED(k_out); NEED(v_out);
  if (dt != VDN_F32 && dt != VDN_BF16) return fail(VDN_ERR_UNSUPPORTED, "unknown dtype %d", (int)dt);
  const vdn_dims& d = *dims;
  if (d.B < 1 || d.H < 1 || d.F < 1) return fail(VDN_ERR_INVALID_ARG, "B=%d H=%d F=%d must be >= 1", d.B, d.H, d.F);
  if (p->grid_h < 1 || p->grid_w < 1) return fail(VDN_ERR_INVALID_ARG, "grid %dx%d", p->grid_h, p->grid_w);
  if ((long long)p->grid_h * p->grid_w != d.N)
    return fail(VDN_ERR_INVALID_ARG, "N=%d != grid_h*grid_w=%d*%d", d.N, p->grid_h, p->grid_w);
  if (d.d_k != d.d_v) return fail(VDN_ERR_UNSUPPORTED, "d_k=%d != d_v=%d", d.d_k, d.d_v);
  if (d.d_k != 16 && d.d_k != 32 && d.d_k != 64 && d.d_k != 128)
    return fail(VDN_ERR_UNSUPPORTED, "head dim %d not in {16,32,64,128}", d.d_k);
  if (p->kernel_h < 1 || p->kernel_h > 7 || p->kernel_h % 2 == 0 || p->kernel_w < 1 || p->kernel_w > 7 ||
      p->kernel_w % 2 == 0)
    return fail(VDN_ERR_UNSUPPORTED, "spatial filter %dx%d: sides must be odd and <= 7", p->kernel_h, p->kernel_w);
  if (p->taps < 1 || p->taps > 5) return fail(VDN_ERR_UNSUPPORTED, "taps=%d not in [1,5]", p->taps);
  if (p->causal != 0 && p->causal != 1) return fail(VDN_ERR_INVALID_ARG, "causal=%d must be 0 or 1", p->causal);
  if (!(p->l2_eps >= 0.f) || !isfinite(p->l2_eps)) return fail(VDN_ERR_INVALID_ARG, "l2_eps must be finite and >= 0");
  const long long L = (long long)d.F * d.N;
  if (L > (1ll << 31) - 1 || (long long)d.B * L * d.H > (1ll << 40))
    return fail(VDN_ERR_INVALID_ARG, "sequence too long (L=%lld)", L);
  if ((long long)d.N * d.H * d.d_k * (dt == VDN_BF16 ? 2 : 4) > 0x7FFFFFF0ll)
    return fail(VDN_ERR_UNSUPPORTED, "one frame of all heads (N=%d H=%d d=%d) exceeds 2 GiB", d.N, d.H, d.d_k);
  if (vdn::prep_tile_cols(d.d_k, p->kernel_h, p->kernel_w, p->grid_w) <= 0)
    return fail(VDN_ERR_UNSUPPORTED, "filter %dx%d does not fit the kernel's LDS tile", p->kernel_h, p->kernel_w);
  hipStream_t s = (hipStream_t)stream;
  if (dt == VDN_BF16)
    VDN_HIP(vdn::launch_vda_prep<uint16_t>(q, k, v, w_spatial, w_temporal, q_out, k_out, v_out, d.B, d.H,
                                           d.F, p->grid_h, p->grid_w, d.d_k, p->kernel_h, p->kernel_w,
                                           p->taps, p->causal, p->l2_eps, s));
  else
    VDN_HIP(vdn::launch_vda_prep<float>(q, k, v, w_spatial, w_temporal, q_out, k_out, v_out, d.B, d.H,
                                        d.F, p->grid_h, p->grid_w, d.d_k, p->kernel_h, p->kernel_w,
                                        p->taps, p->causal, p->l2_eps, s));
  return VDN_OK;
}

}  // extern "C"
