// Host-visible kernel launchers of the VDN library (internal; not the C-ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace vdn {

// Frame geometry of one call.  D = d_k = d_v.
struct Geometry {
  int B, H, F, N, T, D;
  int cf;        // chunk_frames
  int wc;        // window_chunks
  int anchors;   // 0 / 1
  int C;         // F / cf
  long long L;   // F * N
  int Ts;        // text keys inside the Softmax branch (0 = video keys only)
};

// Where query frame t reads the chunk-boundary states and its decay bridge:
// P_fwd[i_f] decayed over frames ws..t and P_rev[i_r] over t..we.  A
// non-anchor frame in chunk c reads the states just outside its window
// (i_f = max(c - wc, 0), i_r = min(c + wc + 1, C)); an anchor frame reads
// the text-only ends (0 and C) over the whole clip.
__host__ __device__ inline void readout_indices(const Geometry& g, int t, int& i_f, int& ws,
                                                int& i_r, int& we) {
  if (g.anchors && (t == 0 || t == g.F - 1)) {
    i_f = 0; ws = 0; i_r = g.C; we = g.F - 1;
    return;
  }
  const int c = t / g.cf;
  i_f = c - g.wc < 0 ? 0 : c - g.wc;
  ws = i_f * g.cf;
  i_r = c + g.wc + 1 > g.C ? g.C : c + g.wc + 1;
  we = (i_r * g.cf < g.F ? i_r * g.cf : g.F) - 1;
}

// Column pitch of the transposed values V^T [D, Lp] of one head on the MFMA
// Softmax path: the L video keys, then the Ts text keys, zero-padded to a
// multiple of 16 columns.
inline long long softmax_vt_pitch(const Geometry& g) {
  return g.L + (g.Ts > 0 ? ((long long)g.Ts + 15) / 16 * 16 : 0);
}

// Work split of the window Softmax over query groups (window_work() in
// window_items.h).
struct SoftmaxWork {
  int GA, GC;    // anchor-frame groups, chunk groups
  int tA, tC;    // query tiles per anchor group / chunk group
  int pa, pc;    // groups per XCD slice
  int grid;      // total workgroups
};

constexpr int kNumXcd = 8;   // MI355X: 8 XCDs, workgroups dealt round-robin

// Query rows per workgroup of the forward window Softmax kernels.
constexpr int kWinMfmaBQ = 256;   // bf16 MFMA kernel: 8 waves x 32 queries
constexpr int kWinSimtBQ = 128;   // generic kernel: one thread per query

// ---- window Softmax (Softmax branch) ----
// q,k [B,H,L,D]; k_text [B,H,Ts,D] (read only when Ts > 0); vt [B,H,D,Lp]
// (bf16 path only, Lp = softmax_vt_pitch); out [B,L,H,D]; lse [B,H,L].
//
// Batched transpose: src [batch][src_rows][cols] -> dst [batch][cols][rows]
// with dst row pitch ldd and batch stride dst_bstride (elements); source rows
// src_rows .. rows-1 are written as zeros.
hipError_t launch_transpose_bf16(const uint16_t* src, uint16_t* dst, long long rows,
                                 long long src_rows, int cols, long long ldd,
                                 long long dst_bstride, long long batch, hipStream_t s);
hipError_t launch_window_softmax_mfma(const Geometry& g, const uint16_t* q, const uint16_t* k,
                                      const uint16_t* k_text, const uint16_t* vt,
                                      const float* g_s, uint16_t* out, float* lse, float scale,
                                      hipStream_t s);
template <typename T>
hipError_t launch_window_softmax_simt(const Geometry& g, const T* q, const T* k, const T* v,
                                      const T* k_text, const T* v_text, const float* g_s, T* out,
                                      float* lse, float scale, hipStream_t s);
bool window_softmax_mfma_ok(const Geometry& g);

// ---- VDA frame statistics + solve (per frame and the text frame) ----
// Tf [B,H,F,D,D], Uf [B,H,F,D,D], S_text [B,H,D,D] (all fp32); Xf (nullable)
// [B,H,F+1,D,D] receives (I + A)^{-1} of every non-anchor frame and of the
// text frame (index F).
template <typename T>
hipError_t launch_vda_frame_solve(const Geometry& g, const T* k, const T* v, const float* beta,
                                  const float* alpha, const T* k_text, const T* v_text,
                                  const float* beta_text, float* Tf, float* Uf, float* S_text,
                                  hipStream_t s, float* Xf = nullptr);

// ---- chunk composition and chunk prefix scans ----
// Tc, Uc [B,H,2,C,D,D] (dir 0 = forward, 1 = reverse)
hipError_t launch_vda_chunk_compose(const Geometry& g, const float* Tf, const float* Uf,
                                    float* Tc, float* Uc, int dirs_mask, hipStream_t s);
// P [B,H,C+1,D,D] for each requested direction (nullable).
// Frame-level scans from the frame maps directly (D = 64, 128 only).
hipError_t launch_vda_frame_scan(const Geometry& g, const float* Tf, const float* Uf,
                                 const float* S_text, float init_scale, float* P_fwd, float* P_rev,
                                 hipStream_t s);
hipError_t launch_vda_chunk_scan(const Geometry& g, const float* Tc, const float* Uc,
                                 const float* S_text, float init_scale, float* P_fwd,
                                 float* P_rev, hipStream_t s);

// ---- readout: gather + decay bridge + q.M + RMSNorm + gate ----
// out [B,L,H,D] (element type T)
template <typename T>
hipError_t launch_vda_readout(const Geometry& g, const T* q, const float* alpha,
                              const float* P_fwd, const float* P_rev, const float* g_l,
                              const float* gamma, float eps, T* out, hipStream_t s);

// ---- linear-branch backward ----
// Workspace and fp32 arguments of launch_vda_bwd (device pointers).  The
// forward recompute (Tf, Uf, Pf, Pr, St, Xf, Tc) must be in place before the
// launch; the rest is scratch or output.  stage 0 launches the readout
// adjoint, stage 1 everything after it.
struct VdaBwdPtrs {
  const float *beta, *alpha, *beta_text, *g_l, *gamma;
  const float *Tf, *Uf, *Pf, *Pr, *St, *Xf, *Tc;
  float *G, *Dbr, *dDbr, *dgp, *dP, *mu, *Sst, *Zst, *ZT, *Rscr;
  float *dbeta, *dalpha, *dbeta_text, *dg_l, *dgamma;
};
template <typename T>
hipError_t launch_vda_bwd(const Geometry& g, const VdaBwdPtrs& p, const T* q, const T* k, const T* v,
                          const T* k_text, const T* v_text, const T* d_out, T* dq, T* dk, T* dv,
                          T* dk_text, T* dv_text, float eps, float init_scale, int stage,
                          hipStream_t s);

// ---- merge ----
// out[M,Dm] = A0[M,K] W0[K,Dm] + A1[M,K] W1[K,Dm]   (bf16 path via W^T)
hipError_t launch_merge_gemm_bf16(const uint16_t* a0, const uint16_t* a1, const uint16_t* w0t,
                                  const uint16_t* w1t, uint16_t* out, long long M, int K, int Dm,
                                  hipStream_t s);
template <typename T>
hipError_t launch_merge_gemm_simt(const T* a0, const T* a1, const T* w0, const T* w1, T* out,
                                  long long M, int K, int Dm, hipStream_t s);
template <typename T>
hipError_t launch_add(const T* a, const T* b, T* out, long long n, hipStream_t s);

// ---- window Softmax backward ----
// o, dout [B,L,H,D] (ungated output and the gradient of the gated output);
// do_hm [B,H,L,D] = g_s * dout; Dq [B,H,L] = g_s * rowsum(dout * o); dg nullable.
template <typename T>
hipError_t launch_softmax_bwd_prep(const Geometry& g, const T* o, const T* dout, const float* g_s,
                                   T* do_hm, float* Dq, float* dg, hipStream_t s);
// Text keys of the backward (g.Ts > 0): k_text, v_text [B,H,Ts,D] (storage
// type of the call) are keys of every query; dk_text, dv_text [B,H,Ts,D]
// receive their gradients.
struct SoftmaxBwdText {
  const void* k_text = nullptr;
  const void* v_text = nullptr;
  void* dk_text = nullptr;
  void* dv_text = nullptr;
};
// q, k, v, do_hm [B,H,L,D]; lse, Dq [B,H,L]; dq, dk, dv [B,H,L,D].
template <typename T>
hipError_t launch_softmax_bwd_simt(const Geometry& g, const T* q, const T* k, const T* v,
                                   const T* do_hm, const float* lse, const float* Dq, T* dq, T* dk,
                                   T* dv, const SoftmaxBwdText& tx, float scale, hipStream_t s);

// bf16 MFMA path (D = 64, 128; N % 16 == 0).
bool softmax_bwd_mfma_ok(const Geometry& g);
hipError_t launch_softmax_bwd_mfma(const Geometry& g, const uint16_t* q, const uint16_t* k,
                                   const uint16_t* v, const uint16_t* do_hm, const float* lse,
                                   const float* Dq, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                                   const SoftmaxBwdText& tx, float scale, hipStream_t s);

// ---- MX-FP8 merge (OCP MX: blocks of 32 along rows, E8M0 scales, E4M3) ----
// src bf16 [rows, cols] -> codes[r * dst_ld + dst_col0 + c], scales[r * dst_ld/32 + (dst_col0 + c)/32].
hipError_t launch_mx_quant_rows(const uint16_t* src, long long rows, int cols, uint8_t* codes,
                                uint8_t* scales, long long dst_ld, int dst_col0, hipStream_t s);
// out[M, Dm] (bf16) = A[M, K2] B^T with A, B^T [Dm, K2] as codes + scales (K2 % 128 == 0).
hipError_t launch_merge_gemm_mx(const uint8_t* a, const uint8_t* a_sc, const uint8_t* bt,
                                const uint8_t* b_sc, uint16_t* out, long long M, int K2, int Dm,
                                hipStream_t s);

// ---- VDA-Prep (linear-branch feature map) ----
// q,k,v [B,L,H,D] token-major -> q',k',v' [B,H,L,D]; w_sp [H,D,kh,kw], w_t [H,D,taps].
template <typename T>
hipError_t launch_vda_prep(const void* q, const void* k, const void* v, const float* w_sp,
                           const float* w_t, void* q_out, void* k_out, void* v_out, int B, int H,
                           int F, int gh, int gw, int D, int kh, int kw, int taps, int causal,
                           float eps, hipStream_t s);
// Column tile of the K/V kernel for these sizes (0 = unsupported).
int prep_tile_cols(int D, int kh, int kw, int gw);

}  // namespace vdn
