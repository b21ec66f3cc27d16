/*
 * vdn.h -- C-ABI of the MI355X (gfx950) Video DeltaNet attention library.
 *
 * The operator is the video-to-video attention of "Video DeltaNet: A
 * Video-Native Hybrid Attention for Livestream Video Generation" (arXiv
 * 2609.20744): a local window Softmax with two boundary anchors, a
 * bidirectional Video Delta Attention (VDA) linear memory started from a
 * text state, and a gated merge through separate output projections.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers owned by the caller, dense and
 *    contiguous in the layouts given (row-major, last index fastest).  The
 *    library never allocates device memory: scratch space is the caller's
 *    `workspace` of at least vdn_workspace_bytes() bytes (256-byte aligned).
 *  - Token layout is frame-major: token row l = f*N + n for frame f in
 *    [0,F) and spatial token n in [0,N); L = F*N.
 *  - `dt` gives the element type of q, k, v, k_text, v_text, W_s, W_l, out
 *    and the branch outputs: VDN_F32 (float) or VDN_BF16 (bfloat16).  The
 *    gates beta, alpha, beta_text, g_s, g_l, gamma are always float; all
 *    states (S_text, P_fwd, P_rev) are always float.
 *  - Inputs are read only and may alias each other; outputs must not alias
 *    inputs, each other, or the workspace.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*,
 *    NULL = the legacy default stream); the library does not synchronise.
 *    vdn_attn_fwd may fork one internal stream through events and always
 *    joins it back onto `stream` before returning.
 *  - Every argument check runs on the host before the first HIP call.  A
 *    failing check returns an error code and launches nothing.  The message
 *    of the last error on the calling thread is vdn_last_error().
 *  - Results are deterministic: no floating-point atomics.
 *  - Supported: d_k == d_v in {16, 32, 64, 128}; F >= 2; F % chunk_frames
 *    == 0; 1 <= N; 0 <= T; B, H >= 1.  Other shapes return
 *    VDN_ERR_INVALID_ARG or VDN_ERR_UNSUPPORTED.
 */
#ifndef VDN_H_
#define VDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VDN_OK = 0,
  VDN_ERR_INVALID_ARG = -1,   /* null pointer, bad size or inconsistent shape */
  VDN_ERR_UNSUPPORTED = -2,   /* valid but not implemented (head dim, dtype)  */
  VDN_ERR_WORKSPACE = -3,     /* workspace smaller than vdn_workspace_bytes() */
  VDN_ERR_HIP = -4,           /* a HIP runtime call or kernel launch failed   */
  /* range anchors, not codes: they give the type the range of int */
  VDN_STATUS_INT_MIN_ = -2147483647 - 1, VDN_STATUS_INT_MAX_ = 2147483647
} vdn_status;

/* The range anchors are not dtypes: they make every int a valid value of the
 * type, so an unknown code passed across the C-ABI is an ordinary value that
 * the library rejects (VDN_ERR_UNSUPPORTED), not undefined behaviour. */
typedef enum {
  VDN_F32 = 0,
  VDN_BF16 = 1,
  VDN_DTYPE_INT_MIN_ = -2147483647 - 1,
  VDN_DTYPE_INT_MAX_ = 2147483647
} vdn_dtype;

/* Problem sizes.  L = F*N video tokens per (b, h); D is the model width of
 * the projected output (D must equal H*d_v when no projections are given). */
typedef struct {
  int B, H, F, N, T, d_k, d_v, D;
} vdn_dims;

/* Operator hyper-parameters; vdn_default_params() fills the page's values.
 *  softmax_scale   : logit scale; <= 0 selects 1/sqrt(d_k) (not printed on
 *                    the page; the standard choice).
 *  rms_eps         : epsilon of the RMSNorm on the linear readout (1e-6).
 *  text_init_scale : each directional scan starts from this multiple of the
 *                    text state; 0.5 makes the two summed readouts count the
 *                    prompt exactly once (method, bidirectional linear
 *                    attention).
 *  chunk_frames    : latent frames per VAE temporal chunk (5).
 *  window_chunks   : a query chunk sees this many chunks on each side (1).
 *  anchors         : 1 = frames 0 and F-1 are boundary anchors with
 *                    four-way connectivity, 0 = no anchors.
 *  text_softmax    : 0 = the Softmax branch sees video keys only (the
 *                    video-to-video operator, default); 1 = the T text
 *                    tokens are keys of every video query too, always
 *                    visible, inside the same softmax (method, bidirectional
 *                    linear attention: the prompt stays directly visible to
 *                    the Softmax branch).  The linear branch is unchanged.
 *  merge_mxfp8     : 0 = the merge GEMM in bf16 with fp32 accumulation
 *                    (default); 1 = both merge operands in MX-FP8 (system
 *                    section: MXFP8 for the wide output GEMMs, states in
 *                    FP32): OCP MX blocks of 32 along the contraction index,
 *                    E8M0 scale 2^(floor(log2 amax) - 8), E4M3 elements
 *                    rounded to nearest even and saturated at 448, fp32
 *                    accumulation.  A reduced-precision mode: bf16 storage
 *                    and the projections W_s, W_l only, H*d_v % 64 == 0,
 *                    D % 8 == 0 (else VDN_ERR_UNSUPPORTED). */
typedef struct {
  float softmax_scale;
  float rms_eps;
  float text_init_scale;
  int chunk_frames;
  int window_chunks;
  int anchors;
  int text_softmax;
  int merge_mxfp8;
} vdn_params;

/* Fills *p with the defaults listed above. */
void vdn_default_params(vdn_params* p);

/*
 * vdn_attn_fwd -- the whole VDN attention forward.
 *
 * Method, hybrid attention (paper: local Softmax window and boundary
 * anchors; bidirectional linear attention; branch calibration):
 *   Ohat_s = g_s * Softmax-window/anchor attention(q, k, v)
 *            (plus the text keys when p->text_softmax = 1)
 *   Ohat_l = g_l * gamma * O_l / sqrt(mean_dv(O_l^2) + rms_eps),
 *            O_l = q^T (M_fwd + M_rev), the two VDA directional memories
 *   out    = Ohat_s W_s + Ohat_l W_l      (heads concatenated, h*d_v + j)
 *
 *  q, k, v     [B,H,L,d]   dt      queries/keys/values, frame-major
 *  beta        [B,H,L]     float   VDA write gate per token (>= 0)
 *  alpha       [B,H,F,d_k] float   VDA channel-wise decay per frame, (0,1]
 *  k_text, v_text [B,H,T,d] dt     text tokens (may be NULL when T == 0)
 *  beta_text   [B,H,T]     float   write gate of the text tokens
 *  g_s, g_l    [B,H,L]     float   post-sigmoid output gates
 *  gamma       [d_v]       float   RMSNorm weight; NULL = all ones
 *  W_s, W_l    [H*d_v, D]  dt      output projections; both NULL = identity
 *                                  (then D == H*d_v and out = Ohat_s+Ohat_l)
 *  out         [B,L,D]     dt
 *  ohat_s, ohat_l [B,L,H,d_v] dt   optional: if non-NULL the gated branch
 *                                  outputs are written there as well.
 */
vdn_status vdn_attn_fwd(const void* q, const void* k, const void* v,
                        const float* beta, const float* alpha,
                        const void* k_text, const void* v_text, const float* beta_text,
                        const float* g_s, const float* g_l, const float* gamma,
                        const void* W_s, const void* W_l,
                        void* out, void* ohat_s, void* ohat_l,
                        void* workspace, size_t workspace_bytes,
                        const vdn_dims* dims, const vdn_params* p, vdn_dtype dt,
                        void* stream);

/*
 * vda_scan_fwd -- forward VDA scan, read at chunk boundaries.
 *
 * Paper, Video Delta Attention (joint frame objective and its closed form)
 * and system section (chunk-wise scans; the prompt state as a leading
 * virtual frame; the small-matrix inverse in FP32):
 *   A_f = K_f^T diag(beta_f) K_f,  W_f = K_f^T diag(beta_f) V_f,
 *   T_f = (I + A_f)^{-1} diag(alpha_f),  U_f = (I + A_f)^{-1} W_f,
 *   anchor frames (when enabled) decay only: T_f = diag(alpha_f), U_f = 0,
 *   S_text = (I + A_text)^{-1} W_text,
 *   P_fwd[0] = text_init_scale * S_text,
 *   P_fwd[c+1] = (maps of frames c*cf .. c*cf+cf-1 applied in order) P_fwd[c].
 *
 *  k, v [B,H,L,d] dt; beta [B,H,L]; alpha [B,H,F,d_k]; text as above.
 *  P_fwd      [B,H,C+1,d_k,d_v] float   (C = F / chunk_frames)
 *  S_text_out [B,H,d_k,d_v]     float   nullable
 */
vdn_status vda_scan_fwd(const void* k, const void* v, const float* beta, const float* alpha,
                        const void* k_text, const void* v_text, const float* beta_text,
                        float* P_fwd, float* S_text_out,
                        void* workspace, size_t workspace_bytes,
                        const vdn_dims* dims, const vdn_params* p, vdn_dtype dt,
                        void* stream);

/*
 * vda_scan_rev -- reverse VDA scan with the same per-frame maps:
 *   P_rev[C] = text_init_scale * S_text,
 *   P_rev[c] = (maps of frames c*cf+cf-1 .. c*cf applied in that order) P_rev[c+1],
 * so P_rev[c] summarises frames >= c*cf.  Arguments as vda_scan_fwd.
 */
vdn_status vda_scan_rev(const void* k, const void* v, const float* beta, const float* alpha,
                        const void* k_text, const void* v_text, const float* beta_text,
                        float* P_rev, float* S_text_out,
                        void* workspace, size_t workspace_bytes,
                        const vdn_dims* dims, const vdn_params* p, vdn_dtype dt,
                        void* stream);

/*
 * vdn_window_softmax_fwd -- the Softmax branch alone.
 *
 * Paper, method, local Softmax window: query frame t in chunk c sees every
 * token of the frames whose chunk is within window_chunks of c, plus (with
 * anchors) frames 0 and F-1; frames 0 and F-1 see every frame; each frame is
 * counted once.  out = g_s * softmax(scale * q k^T) v over those keys.
 * With p->text_softmax = 1 the dims->T text tokens join every query's keys.
 *
 *  q, k, v [B,H,L,d] dt;  g_s [B,H,L] float, NULL = 1
 *  k_text, v_text [B,H,T,d] dt   read only when p->text_softmax = 1 and
 *                                T > 0 (then non-NULL), else may be NULL
 *  out [B,L,H,d_v] dt;  lse [B,H,L] float natural-log normaliser, nullable
 */
vdn_status vdn_window_softmax_fwd(const void* q, const void* k, const void* v,
                                  const void* k_text, const void* v_text, const float* g_s,
                                  void* out, float* lse,
                                  void* workspace, size_t workspace_bytes,
                                  const vdn_dims* dims, const vdn_params* p, vdn_dtype dt,
                                  void* stream);

/*
 * vdn_window_softmax_fwd_noalloc -- vdn_window_softmax_fwd for callers that
 * cannot allocate (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): no workspace argument and no device
 * allocation.  Its scratch (V^T and the text values of the bf16 MFMA path,
 * vdn_softmax_workspace_bytes() of them) lives in a device array of the
 * library of at most 64 MiB, one per GPU, held until the process ends.
 *  Arguments, outputs and results as vdn_window_softmax_fwd (same kernels).
 *  Sizes whose scratch exceeds 64 MiB: VDN_ERR_UNSUPPORTED, nothing launched.
 *  Every call on one GPU shares that array: calls that overlap on one GPU
 *  (on different streams or threads without ordering) race.  Each call
 *  rewrites every scratch element it reads, so no clearing is needed.
 */
vdn_status vdn_window_softmax_fwd_noalloc(const void* q, const void* k, const void* v,
                                          const void* k_text, const void* v_text,
                                          const float* g_s, void* out, float* lse,
                                          const vdn_dims* dims, const vdn_params* p,
                                          vdn_dtype dt, void* stream);

/*
 * vdn_merge_fwd -- the merge alone (step a8 of vdn_attn_fwd).
 *
 * Paper, method, branch calibration: each branch has its own output
 * projection and the projected outputs are added:
 *   out = Ohat_s W_s + Ohat_l W_l       (heads concatenated, h*d_v + j)
 * in bf16 with fp32 accumulation, or in MX-FP8 with p->merge_mxfp8 = 1
 * (system section, other optimizations).  Only dims->B, H, F, N, d_k, d_v
 * and D are used (L = F*N tokens); the other fields must still be valid.
 *
 *  ohat_s, ohat_l [B,L,H,d_v] dt;  W_s, W_l [H*d_v, D] dt, both NULL = identity
 *  out [B,L,D] dt;  workspace of vdn_workspace_bytes(dims, p, dt) bytes
 */
vdn_status vdn_merge_fwd(const void* ohat_s, const void* ohat_l, const void* W_s, const void* W_l,
                         void* out, void* workspace, size_t workspace_bytes,
                         const vdn_dims* dims, const vdn_params* p, vdn_dtype dt, void* stream);

/*
 * vdn_merge_bwd -- gradients of the merge (a8).
 *
 * Paper, method, branch calibration defines out = Ohat_s W_s + Ohat_l W_l
 * (heads concatenated); the experiments train through it.  For the output
 * gradient d_out the gradients of the two matrix products are
 *   d_ohat_s = d_out W_s^T,  d_ohat_l = d_out W_l^T,
 *   dW_s = Ohat_s^T d_out,   dW_l = Ohat_l^T d_out    (summed over all B*L tokens),
 * in bf16 with fp32 accumulation.  Without projections (W_s = W_l = NULL,
 * out = Ohat_s + Ohat_l) d_ohat_s = d_ohat_l = d_out.  Only dims->B, H, F,
 * N, d_k, d_v and D are used.
 *
 *  ohat_s, ohat_l [B,L,H,d_v] dt   the forward's branch outputs (read only for dW)
 *  W_s, W_l       [H*d_v, D]  dt   or both NULL
 *  d_out          [B,L,D]     dt
 *  d_ohat_s, d_ohat_l [B,L,H,d_v] dt  outputs
 *  dW_s, dW_l     [H*d_v, D]  dt   outputs, or both NULL to skip the weight gradients
 *  workspace      vdn_merge_bwd_workspace_bytes(dims, p, dt) bytes (used only for dW)
 * Errors: VDN_ERR_UNSUPPORTED with projections unless dt is bf16, D % 128 == 0,
 * H*d_v % 8 == 0, each operand below 2 GiB and, for dW, B*L % 128 == 0;
 * VDN_ERR_INVALID_ARG for NULL required pointers or an unpaired W / dW;
 * VDN_ERR_WORKSPACE for a short workspace.
 */
vdn_status vdn_merge_bwd(const void* ohat_s, const void* ohat_l, const void* W_s, const void* W_l,
                         const void* d_out, void* d_ohat_s, void* d_ohat_l, void* dW_s, void* dW_l,
                         void* workspace, size_t workspace_bytes, const vdn_dims* dims,
                         const vdn_params* p, vdn_dtype dt, void* stream);
/* Workspace bytes of vdn_merge_bwd (0 if the arguments are invalid). */
size_t vdn_merge_bwd_workspace_bytes(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt);

/*
 * vdn_window_softmax_bwd -- gradients of the Softmax branch (a7).
 *
 * Paper, method (local Softmax window; branch calibration) defines the
 * forward Ohat_s = g_s * softmax(scale q k^T) v over the visible keys; the
 * experiments train through it.  The gradients are its chain rule:
 *   dO = g_s * d_out,  Dq = rowsum(dO * o),  P = exp(scale q.k - lse),
 *   dS = P * (dO.v - Dq),  dq = scale * sum_k dS k,  dk = scale * sum_q dS q,
 *   dv = sum_q P dO,  dg_s = rowsum(d_out * o).
 * With p->text_softmax = 1 and dims->T > 0 (method, bidirectional linear
 * attention: the text stays visible to the Softmax branch) the T text tokens
 * are keys of every query in the same softmax, and their gradients are
 * summed over all queries.
 *
 *  q, k, v     [B,H,L,d] dt     the forward's inputs
 *  k_text, v_text [B,H,T,d] dt  the text keys and values (read only with text keys)
 *  o           [B,L,H,d] dt     the ungated Softmax output O_s
 *                               (vdn_window_softmax_fwd with g_s = NULL, same p)
 *  lse         [B,H,L]   float  the forward's log-sum-exp (same call)
 *  g_s         [B,H,L]   float  the gate, NULL = 1
 *  d_out       [B,L,H,d] dt     gradient of the gated output Ohat_s
 *  dq, dk, dv  [B,H,L,d] dt     outputs (fully written)
 *  dk_text, dv_text [B,H,T,d] dt  outputs with text keys (fully written), else unused
 *  dg_s        [B,H,L]   float  output gradient of g_s, nullable
 *  workspace   vdn_softmax_bwd_workspace_bytes(dims, p, dt) bytes
 * Errors: VDN_ERR_INVALID_ARG for a NULL required pointer (k_text, v_text,
 * dk_text, dv_text are required with text keys) or invalid dims;
 * VDN_ERR_WORKSPACE for a short workspace.
 */
vdn_status vdn_window_softmax_bwd(const void* q, const void* k, const void* v,
                                  const void* k_text, const void* v_text, const void* o,
                                  const float* lse, const float* g_s, const void* d_out, void* dq,
                                  void* dk, void* dv, void* dk_text, void* dv_text, float* dg_s,
                                  void* workspace, size_t workspace_bytes, const vdn_dims* dims,
                                  const vdn_params* p, vdn_dtype dt, void* stream);

/* Workspace bytes of vdn_window_softmax_bwd (0 if the arguments are invalid). */
size_t vdn_softmax_bwd_workspace_bytes(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt);

/*
 * vda_bwd -- gradients of the linear (VDA) branch output Ohat_l with respect
 * to every input of the branch.
 *
 * Paper: the Video Delta Attention section (frame statistics A = K^T B K,
 * W = K^T B V and the frame update S_f = (I + A_f)^{-1}(diag(alpha_f) S_{f-1}
 * + W_f)), the method's bidirectional linear attention (text-initialised
 * scans, gather + decay bridge, sum of the two readouts) and branch
 * calibration (RMSNorm + gate) define the forward of vdn_attn_fwd's linear
 * branch; the experiments train through it.  These are its chain-rule
 * gradients.  The call recomputes the forward scans itself (nothing from a
 * forward call is needed).
 *
 *  q, k, v               [B,H,L,d] dt     the forward's inputs
 *  beta, g_l             [B,H,L]   float
 *  alpha                 [B,H,F,d] float  decay gates, in (0, 1]
 *  k_text, v_text        [B,H,T,d] dt     (required when T > 0)
 *  beta_text             [B,H,T]   float  (required when T > 0)
 *  gamma                 [d]       float  RMSNorm weight, NULL = 1
 *  d_out                 [B,L,H,d] dt     gradient of Ohat_l
 *  dq, dk, dv            [B,H,L,d] dt     outputs, fully written (zero dk,
 *                                          dv, dbeta on anchor frames, which
 *                                          the scans do not write)
 *  dbeta                 [B,H,L]   float  output
 *  dalpha                [B,H,F,d] float  output
 *  dk_text, dv_text      [B,H,T,d] dt     outputs (required when T > 0)
 *  dbeta_text            [B,H,T]   float  output (required when T > 0)
 *  dg_l                  [B,H,L]   float  output, nullable
 *  dgamma                [d]       float  output, nullable (summed over
 *                                          batch, heads and tokens)
 *  workspace             vda_bwd_workspace_bytes(dims, p, dt) bytes
 * Errors as for vdn_attn_fwd; F > 1024 -> VDN_ERR_UNSUPPORTED.  Deterministic
 * (no atomics).
 */
vdn_status vda_bwd(const void* q, const void* k, const void* v, const float* beta,
                   const float* alpha, const void* k_text, const void* v_text,
                   const float* beta_text, const float* g_l, const float* gamma, const void* d_out,
                   void* dq, void* dk, void* dv, float* dbeta, float* dalpha, void* dk_text,
                   void* dv_text, float* dbeta_text, float* dg_l, float* dgamma, void* workspace,
                   size_t workspace_bytes, const vdn_dims* dims, const vdn_params* p, vdn_dtype dt,
                   void* stream);

/* Workspace bytes of vda_bwd (0 if the arguments are invalid). */
size_t vda_bwd_workspace_bytes(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt);

/*
 * vdn_mx_quantize -- MX-FP8 quantization of bf16 rows (the operand format of
 * the MX-FP8 merge; e.g. to inspect it or to quantize weights ahead of time).
 *
 * OCP Microscaling (MX) v1.0 with E4M3 elements: each block of 32
 * consecutive elements of a row gets scale byte s + 127 with
 * s = floor(log2(max |x|)) - 8 clamped to [-127, 127] (s = -127 for a zero
 * block), and codes[i] = E4M3(x[i] / 2^s), rounded to nearest even, with
 * magnitudes >= 448 saturated to 448 and the sign of x kept.
 *
 *  src    [rows, cols] bf16 (device);  cols % 32 == 0
 *  codes  [rows, cols] uint8 (device);  scales [rows, cols/32] uint8 (device)
 */
vdn_status vdn_mx_quantize(const void* src, void* codes, void* scales, long long rows, int cols,
                           void* stream);

/*
 * vda_prep_fwd -- VDA-Prep, the linear branch's feature map (upstream of
 * vdn_attn_fwd's linear-branch inputs).
 *
 * Paper, method (the two branches): the linear branch applies a separable
 * short convolution to K and V -- a depthwise spatial filter and a five-tap
 * temporal filter -- then SiLU, and L2-normalises Q and K; system section
 * (fused VDA kernels): VDA-Prep fuses the temporal convolution, SiLU, L2
 * normalisation and the conversion to the frame-major layout.
 *   conv(x)[f,y,x,c] = sum_tau w_temporal[h,c,tau] sum_{dy,dx} w_spatial[h,c,dy,dx]
 *                      * x[f+tau-t0, y+dy-(kernel_h-1)/2, x+dx-(kernel_w-1)/2, c]
 *     with zeros outside the clip and the grid; t0 = (taps-1)/2 (centred) or
 *     taps-1 (causal);
 *   q' = q / sqrt(|q|^2 + l2_eps),  k' = L2(SiLU(conv(k))),  v' = SiLU(conv(v)),
 *     norms over the d channels of one token of one head.
 *
 *  q, k, v             [B,L,H,d] dt   token-major projection outputs; token n
 *                                     of a frame sits at grid row n / grid_w,
 *                                     column n % grid_w (N = grid_h * grid_w)
 *  w_spatial           [H,d,kernel_h,kernel_w] float   depthwise spatial filter
 *  w_temporal          [H,d,taps]  float   depthwise temporal filter
 *  q_out, k_out, v_out [B,H,L,d]   dt     frame-major, head-major features
 * Uses dims B, H, F, N and d_k (== d_v); T and D are ignored; F >= 1.  No
 * workspace.  Supported: d in {16,32,64,128}; kernel_h, kernel_w odd in [1,7];
 * taps in [1,5]; one frame of all heads (N * H * d elements) at most 2 GiB
 * (VDN_ERR_UNSUPPORTED otherwise).  Outputs must not alias inputs.
 */
typedef struct {
  int grid_h, grid_w;      /* latent grid of one frame, N = grid_h * grid_w          */
  int kernel_h, kernel_w;  /* spatial filter size (odd); not printed on the page: 3x3 */
  int taps;                /* temporal filter taps (5)                               */
  int causal;              /* 0 = centred taps, 1 = taps end at the output frame     */
  float l2_eps;            /* epsilon under the L2 norm's square root (1e-6)         */
} vda_prep_params;

/* Fills *p: the given grid, 3x3 spatial filter, 5 centred taps, eps 1e-6. */
void vda_prep_default_params(vda_prep_params* p, int grid_h, int grid_w);

vdn_status vda_prep_fwd(const void* q, const void* k, const void* v,
                        const float* w_spatial, const float* w_temporal,
                        void* q_out, void* k_out, void* v_out,
                        const vdn_dims* dims, const vda_prep_params* p, vdn_dtype dt,
                        void* stream);

/* Workspace bytes that suffice for every entry point above at these sizes
 * (vdn_attn_fwd's full layout); 0 if the arguments are invalid.  vdn_attn_fwd
 * needs the full amount only when it keeps Ohat_s / Ohat_l in the workspace:
 * with both ohat_s and ohat_l given, those two regions (the last ones) are not
 * required. */
size_t vdn_workspace_bytes(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt);
/* What one entry point alone requires (0 if the arguments are invalid):
 *  vdn_scan_workspace_bytes     vda_scan_fwd / vda_scan_rev: the fp32 frame
 *                               maps T_f, U_f, S_text (+ the chunk maps for
 *                               d = 16, 32)
 *  vdn_softmax_workspace_bytes  vdn_window_softmax_fwd: V^T (and the text
 *                               values) on the bf16 MFMA path, else 0
 *  vdn_merge_workspace_bytes    vdn_merge_fwd: W_s^T, W_l^T (+ MX-FP8 operands) */
size_t vdn_scan_workspace_bytes(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt);
size_t vdn_softmax_workspace_bytes(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt);
size_t vdn_merge_workspace_bytes(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt);

/*
 * vdn_window_plan -- host-only helper: the frame roles the kernels use
 * (method, local Softmax window and boundary anchors; bidirectional linear
 * attention: the states gathered just outside the window and the decay
 * bridge over the skipped span).
 *  vis   [F*F] row = query frame, 1 = key frame visible to Softmax (nullable);
 *        built by running the Softmax kernels' own work-item decoder over
 *        their whole grid (one head, one token per frame)
 *  i_fwd, ws, i_rev, we [F] (each nullable): query frame t reads
 *        P_fwd[i_fwd[t]] decayed over frames ws[t]..t and P_rev[i_rev[t]]
 *        decayed over frames t..we[t]; the readout kernels' own function.
 * Host memory, caller owned.  No device is touched.  Fails with
 * VDN_ERR_UNSUPPORTED if the work items do not cover every query frame
 * exactly once.
 */
vdn_status vdn_window_plan(int F, const vdn_params* p, uint8_t* vis,
                           int32_t* i_fwd, int32_t* ws, int32_t* i_rev, int32_t* we);

/*
 * vdn_window_row_keys -- host-only helper: how many keys each query row's
 * softmax runs over, in the launch vdn_window_softmax_fwd makes for these
 * dims, params and dtype (method, local Softmax window: N tokens of every
 * visible frame, plus the T text keys with text_softmax).  The library runs
 * that launch's work-item decoder over its whole grid on the host.
 *  keys [B*H*L] int64, host memory, caller owned: keys[(b*H + h)*L + l] for
 *       query row l of head (b, h); -1 where the row is covered by no work
 *       item or by more than one.
 * No device is touched.  Argument errors as for vdn_window_softmax_fwd;
 * VDN_ERR_INVALID_ARG if B*H*L exceeds 2^31.
 */
vdn_status vdn_window_row_keys(const vdn_dims* dims, const vdn_params* p, vdn_dtype dt,
                               int64_t* keys);

/*
 * Kernel timer (instrumentation for roofline measurements).
 * vdn_timer_enable(n): the next n launches of the window Softmax kernel made
 *   by this thread (through vdn_attn_fwd or vdn_window_softmax_fwd) are each
 *   bracketed by a pair of HIP events recorded on the stream the kernel runs
 *   on.  The library creates the events (no device memory is allocated).
 * vdn_timer_read(ms, cap): waits for the recorded events and writes up to
 *   cap per-launch durations in milliseconds to host array ms; returns the
 *   number written (negative vdn_status on error).
 * vdn_timer_disable(): stops recording and destroys the events.
 */
vdn_status vdn_timer_enable(int n);
int vdn_timer_read(float* ms, int cap);
void vdn_timer_disable(void);

/* Static text of a status code. */
const char* vdn_status_string(vdn_status s);
/* Message of the last failing call on this thread ("" if none). */
const char* vdn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VDN_H_ */
