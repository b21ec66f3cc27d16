// VDA per-frame statistics and the frame solve.
//
// Paper ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream
// Video Generation"), Video Delta Attention section: a frame's joint update
// solves (I + A_f) S_f = diag(alpha_f) S_{f-1} + W_f with the frame
// statistics A_f = K_f^T diag(beta_f) K_f and W_f = K_f^T diag(beta_f) V_f.
// System section, small-matrix inverse: one kernel performs a blocked
// Gauss-Jordan elimination in registers and directly emits the transition
// T_f = (I + A_f)^{-1} diag(alpha_f) and the injection U_f = (I + A_f)^{-1} W_f,
// in fp32.  The text state is the same solve on the text tokens from a zero
// state (the leading virtual frame): S_text = (I + A_text)^{-1} W_text.
//
// Our design: one workgroup (256 threads) per (b, h, frame), frame index F
// being the text frame.  I + A is symmetric positive definite (eigenvalues
// >= 1), so the elimination needs no pivoting.
//
// bf16 kernel (D = 64, 128): statistics on v_mfma_f32_32x32x16_bf16 and a
// blocked Gauss-Jordan (16-column panels factored in registers, rank-16
// trailing updates on v_mfma_f32_32x32x2f32), both in one block ownership of
// [I + A | W] (see the kernel).  Tokens must be the contracted
// (lane-contiguous) index of the statistics, so each 64-token tile is
// transposed into LDS ([channel][token]).  beta * K is formed in fp32 and
// split into bf16 hi + lo parts, so A and W carry ~16 more mantissa bits than
// a single bf16 product.
//
// Generic kernel (fp32 storage, any D): fp32 VALU statistics and an
// unblocked elimination on a 16 x 16 thread grid (thread (tr, tc) owns an
// 8 x 8 block of both halves; one barrier per pivot).
#include "vdn_common.h"
#include "vdn_internal.h"

#include <utility>

namespace vdn {

template <typename T>
struct SolveArgs {
  Geometry g;
  const T* k;
  const T* v;
  const float* beta;
  const float* alpha;
  const T* k_text;
  const T* v_text;
  const float* beta_text;
  float* Tf;
  float* Uf;
  float* S_text;
  float* Xf;      // optional: (I + A)^{-1} per frame, text frame last [B,H,F+1,D,D]
};

struct GJShared {
  float colbuf[2][128];
  float rowM[2][128];
  float rowW[2][128];
};

// Anchor frames are excluded from both scans: decay only (T = diag(alpha), U = 0).
template <int D>
__device__ __forceinline__ void emit_anchor(const Geometry& g, const float* alpha, float* Tf,
                                            float* Uf, int bh, int fr) {
  const size_t DD = (size_t)D * D;
  const float* al = alpha + ((size_t)bh * g.F + fr) * D;
  float* Tout = Tf + ((size_t)bh * g.F + fr) * DD;
  float* Uout = Uf + ((size_t)bh * g.F + fr) * DD;
  for (int e = threadIdx.x; e < D * D; e += blockDim.x) {
    const int i = e / D, j = e % D;
    Tout[e] = (i == j) ? al[j] : 0.f;
    Uout[e] = 0.f;
  }
}

// In-place Gauss-Jordan on [I + A | W] held as (m | w) in the thread-grid
// ownership; on return m = (I + A)^{-1} and w = (I + A)^{-1} W.
template <int D>
__device__ __forceinline__ void gauss_jordan(float (&m)[D / 16][D / 16], float (&w)[D / 16][D / 16],
                                             GJShared& sh, int tr, int tc) {
  constexpr int R = D / 16;
  for (int kb = 0; kb < 16; ++kb) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int k = kb * R + r;
      const int buf = k & 1;
      if (tc == kb) {
#pragma unroll
        for (int i = 0; i < R; ++i) sh.colbuf[buf][tr * R + i] = m[i][r];
      }
      if (tr == kb) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
          sh.rowM[buf][tc * R + j] = m[r][j];
          sh.rowW[buf][tc * R + j] = w[r][j];
        }
      }
      __syncthreads();
      const float p = 1.f / sh.rowM[buf][k];
      float cik[R], rkj[R], rkw[R];
#pragma unroll
      for (int i = 0; i < R; ++i) cik[i] = sh.colbuf[buf][tr * R + i] * p;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        rkj[j] = sh.rowM[buf][tc * R + j];
        rkw[j] = sh.rowW[buf][tc * R + j];
      }
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < R; ++j) {
          m[i][j] = fmaf(-cik[i], rkj[j], m[i][j]);
          w[i][j] = fmaf(-cik[i], rkw[j], w[i][j]);
        }
      if (tr == kb) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
          m[r][j] = rkj[j] * p;
          w[r][j] = rkw[j] * p;
        }
      }
      if (tc == kb) {
#pragma unroll
        for (int i = 0; i < R; ++i) m[i][r] = -cik[i];
      }
      if (tr == kb && tc == kb) m[r][r] = p;
    }
  }
}

// Write T = X diag(alpha), U = X W for a video frame, or S_text = X W; and
// X itself when Xf is set (the backward pass solves with it).
template <int D>
__device__ __forceinline__ void emit_solution(const Geometry& g, const float* alpha, float* Tf,
                                              float* Uf, float* S_text, float* Xf, int bh, int fr,
                                              bool text, const float (&m)[D / 16][D / 16],
                                              const float (&w)[D / 16][D / 16], int tr, int tc) {
  constexpr int R = D / 16;
  const size_t DD = (size_t)D * D;
  if (Xf) {
    float* X = Xf + ((size_t)bh * (g.F + 1) + fr) * DD;
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int j = 0; j < R; ++j) X[(size_t)(tr * R + i) * D + tc * R + j] = m[i][j];
  }
  if (text) {
    float* S = S_text + (size_t)bh * DD;
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int j = 0; j < R; ++j) S[(size_t)(tr * R + i) * D + tc * R + j] = w[i][j];
    return;
  }
  const float* al = alpha + ((size_t)bh * g.F + fr) * D;
  float* Tout = Tf + ((size_t)bh * g.F + fr) * DD;
  float* Uout = Uf + ((size_t)bh * g.F + fr) * DD;
  float aj[R];
#pragma unroll
  for (int j = 0; j < R; ++j) aj[j] = al[tc * R + j];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const size_t e = (size_t)(tr * R + i) * D + tc * R + j;
      Tout[e] = m[i][j] * aj[j];
      Uout[e] = w[i][j];
    }
}

// alpha of video frame fr (unused for the text frame, fr == F).
template <typename T>
__device__ __forceinline__ const float* alpha_row(const SolveArgs<T>& a, int bh, int fr) {
  return a.alpha + ((size_t)bh * a.g.F + (fr < a.g.F ? fr : 0)) * a.g.D;
}

template <typename T>
__device__ __forceinline__ void frame_tokens(const SolveArgs<T>& a, int bh, int fr, bool text,
                                             const T*& kp, const T*& vp, const float*& bp,
                                             long long& ntok) {
  const Geometry& g = a.g;
  if (text) {
    ntok = g.T;
    kp = a.k_text + (size_t)bh * g.T * g.D;
    vp = a.v_text + (size_t)bh * g.T * g.D;
    bp = a.beta_text + (size_t)bh * g.T;
  } else {
    ntok = g.N;
    const size_t off = (size_t)bh * g.L + (size_t)fr * g.N;
    kp = a.k + off * g.D;
    vp = a.v + off * g.D;
    bp = a.beta + off;
  }
}

// ---------------------------------------------------------------------------
// Generic kernel: fp32 VALU statistics.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void vda_frame_solve_kernel(SolveArgs<T> a) {
  constexpr int R = D / 16;
  constexpr int TT = 32;  // tokens per LDS stage
  __shared__ float Ks[TT][D + 1];
  __shared__ float Vs[TT][D + 1];
  __shared__ float Bs[TT];
  __shared__ GJShared sh;

  const Geometry& g = a.g;
  const int fr = blockIdx.x % (g.F + 1);
  const int bh = blockIdx.x / (g.F + 1);
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  const bool text = (fr == g.F);
  if (!text && g.anchors && (fr == 0 || fr == g.F - 1)) {
    emit_anchor<D>(g, a.alpha, a.Tf, a.Uf, bh, fr);
    return;
  }
  const T *kp, *vp;
  const float* bp;
  long long ntok;
  frame_tokens(a, bh, fr, text, kp, vp, bp, ntok);

  float m[R][R], w[R][R];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < R; ++j) {
      m[i][j] = 0.f;
      w[i][j] = 0.f;
    }
  for (long long t0 = 0; t0 < ntok; t0 += TT) {
    const int nt = (int)min((long long)TT, ntok - t0);
    __syncthreads();
    for (int e = tid; e < TT * D; e += 256) {
      const int r = e / D, c = e % D;
      Ks[r][c] = r < nt ? Elem<T>::load(kp, (size_t)(t0 + r) * D + c) : 0.f;
      Vs[r][c] = r < nt ? Elem<T>::load(vp, (size_t)(t0 + r) * D + c) : 0.f;
    }
    if (tid < TT) Bs[tid] = tid < nt ? bp[t0 + tid] : 0.f;
    __syncthreads();
    for (int r = 0; r < nt; ++r) {
      const float b = Bs[r];
      float kr[R], kc[R], vc[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        kr[i] = b * Ks[r][tr * R + i];
        kc[i] = Ks[r][tc * R + i];
        vc[i] = Vs[r][tc * R + i];
      }
#pragma unroll
      for (int i = 0; i < R; ++i)
#pragma unroll
        for (int j = 0; j < R; ++j) {
          m[i][j] = fmaf(kr[i], kc[j], m[i][j]);
          w[i][j] = fmaf(kr[i], vc[j], w[i][j]);
        }
    }
  }
  if (tr == tc) {
#pragma unroll
    for (int i = 0; i < R; ++i) m[i][i] += 1.f;
  }
  gauss_jordan<D>(m, w, sh, tr, tc);
  emit_solution<D>(g, a.alpha, a.Tf, a.Uf, a.S_text, a.Xf, bh, fr, text, m, w, tr, tc);
}

// ---------------------------------------------------------------------------
// bf16 kernel (D = 64, 128): MFMA statistics and a blocked Gauss-Jordan solve.
//
// Ownership: [I + A | W] is NB x 2NB blocks of 32 x 32 (NB = D / 32).  Wave w
// owns BPW = NB * 2NB / 4 blocks of one block row rb (D = 128: the whole row
// block w; D = 64: half of row block w / 2), as v_mfma 32 x 32 accumulators
// (lane l: column l % 32, rows mfma32_row(i, l / 32)).  The statistics write
// straight into that ownership, and so does the solve.
//
// Solve: panels of PW = 16 columns, left to right.  For panel k (columns
// c0 .. c0 + 15) the in-place elimination of its 16 pivots is a left
// multiplication by a matrix E_k that differs from I only in those columns,
// G_k = E_k[:, panel].  Every wave factors the D x 16 panel redundantly in
// registers (lane = row, pivot rows broadcast with v_readlane; no barrier),
// giving G_k.  Then each wave applies the rank-16 update
//   X[:, j] += (G_k - I_k) X[pivot rows, j]
// to all of its blocks on v_mfma_f32_32x32x2f32; the panel's own columns are
// preset to the identity pattern with B = I there, so they become G_k (the
// in-place inverse).  After the last panel the left half holds
// X = (I + A)^{-1} and the right half X W.  One barrier per panel (panel
// columns and pivot rows are exchanged through double-buffered LDS).
// ---------------------------------------------------------------------------
template <int D>
// Two workgroups per compute unit (at most 256 registers per lane): at
// d = 128 the kernel then spills ~30 registers, and still runs ~20% faster
// than at one workgroup per compute unit, where every wait of the elimination
// leaves its SIMD idle.
__global__ __launch_bounds__(256, 2) void vda_frame_solve_mfma_kernel(SolveArgs<bf16_t> a) {
  constexpr int TT = 64;            // tokens per tile
  constexpr int TP = TT + 8;        // transposed tile pitch (bf16)
  constexpr int NB = D / 32;        // 32-blocks per matrix side
  constexpr int NCB = 2 * NB;       // block columns of [I + A | W]
  constexpr int BPW = NB * NCB / 4; // blocks per wave
  constexpr int PAIRS = TT / 2 * (D / 8) / 256;   // (token pair, 8-channel chunk) per thread
  constexpr int PW = 16;            // panel width
  constexpr int NP = D / PW;        // panels
  constexpr int RS = D / 64;        // rows per lane in the panel factorization
  constexpr int PP = PW + 4;        // LDS pitch of panel rows (floats): conflict-free 16-byte reads
  static_assert(NCB % BPW == 0, "a wave's blocks lie in one block row");
  struct StatsTiles {
    bf16_t kt[D * TP];    // K^T
    bf16_t kh[D * TP];    // (beta K)^T, bf16 high part
    bf16_t kl[D * TP];    // (beta K)^T, bf16 low part
    bf16_t vt[D * TP];    // V^T
  };
  struct SolveTiles {
    float pnl[2][D * PP];        // panel columns, row-major [row][PP]
    float prt[2][NCB * 32 * PP]; // pivot rows, transposed [column][PP], k-slots permuted
  };
  union Smem {
    StatsTiles st;
    SolveTiles sv;
  };
  __shared__ __attribute__((aligned(16))) Smem sm;

  const Geometry& g = a.g;
  const int fr = blockIdx.x % (g.F + 1);
  const int bh = blockIdx.x / (g.F + 1);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hg = lane >> 5, l32 = lane & 31;
  const bool text = (fr == g.F);
  if (!text && g.anchors && (fr == 0 || fr == g.F - 1)) {
    emit_anchor<D>(g, a.alpha, a.Tf, a.Uf, bh, fr);
    return;
  }
  const bf16_t *kp, *vp;
  const float* bp;
  long long ntok;
  frame_tokens(a, bh, fr, text, kp, vp, bp, ntok);

  const int rb = wave * BPW / NCB;            // this wave's block row
  const int cb0 = (wave * BPW) % NCB;         // its first block column
  f32x16 acc[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) acc[i] = f32x16{};

  // raw tile data for (token pair, 8-channel chunk) units, prefetched one
  // tile ahead so the global loads overlap the previous tile's MFMAs
  u32x4 pk_a[PAIRS], pk_b[PAIRS], pv_a[PAIRS], pv_b[PAIRS];
  float pb_a[PAIRS], pb_b[PAIRS];
  auto fetch = [&](long long t0) {
    const int nt = (int)min((long long)TT, ntok - t0);
#pragma unroll
    for (int i = 0; i < PAIRS; ++i) {
      const int pc = tid + 256 * i;
      const int p = pc % (TT / 2), c8 = pc / (TT / 2);
      const int t_a = 2 * p, t_b = 2 * p + 1;
      pk_a[i] = pk_b[i] = pv_a[i] = pv_b[i] = u32x4{0, 0, 0, 0};
      pb_a[i] = pb_b[i] = 0.f;
      if (t_a < nt) {
        pk_a[i] = ld16(kp + (size_t)(t0 + t_a) * D + c8 * 8);
        pv_a[i] = ld16(vp + (size_t)(t0 + t_a) * D + c8 * 8);
        pb_a[i] = bp[t0 + t_a];
      }
      if (t_b < nt) {
        pk_b[i] = ld16(kp + (size_t)(t0 + t_b) * D + c8 * 8);
        pv_b[i] = ld16(vp + (size_t)(t0 + t_b) * D + c8 * 8);
        pb_b[i] = bp[t0 + t_b];
      }
    }
  };
  // transpose into [channel][token], two tokens per 4-byte write
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < PAIRS; ++i) {
      const int pc = tid + 256 * i;
      const int p = pc % (TT / 2), c8 = pc / (TT / 2);
      const int t_a = 2 * p;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const uint32_t sh16 = (jj & 1) * 16;
        const uint32_t xa = (pk_a[i][jj >> 1] >> sh16) & 0xFFFFu, xb = (pk_b[i][jj >> 1] >> sh16) & 0xFFFFu;
        const uint32_t ya = (pv_a[i][jj >> 1] >> sh16) & 0xFFFFu, yb = (pv_b[i][jj >> 1] >> sh16) & 0xFFFFu;
        const float fa = pb_a[i] * bf16_to_f32((bf16_t)xa), fb = pb_b[i] * bf16_to_f32((bf16_t)xb);
        const bf16_t ha = f32_to_bf16(fa), hb = f32_to_bf16(fb);
        const bf16_t la = f32_to_bf16(fa - bf16_to_f32(ha)), lb = f32_to_bf16(fb - bf16_to_f32(hb));
        const int off = (c8 * 8 + jj) * TP + t_a;
        *reinterpret_cast<uint32_t*>(&sm.st.kt[off]) = xa | (xb << 16);
        *reinterpret_cast<uint32_t*>(&sm.st.vt[off]) = ya | (yb << 16);
        *reinterpret_cast<uint32_t*>(&sm.st.kh[off]) = (uint32_t)ha | ((uint32_t)hb << 16);
        *reinterpret_cast<uint32_t*>(&sm.st.kl[off]) = (uint32_t)la | ((uint32_t)lb << 16);
      }
    }
  };

  // ---- statistics: block (rb, cb) of A = (beta K)^T K (cb < NB) or of
  // W = (beta K)^T V (cb >= NB); the A operand (channels of block row rb)
  // is shared by all of the wave's blocks
  if (ntok > 0) fetch(0);
  for (long long t0 = 0; t0 < ntok; t0 += TT) {
    __syncthreads();
    stage();
    __syncthreads();
    if (t0 + TT < ntok) fetch(t0 + TT);
#pragma unroll
    for (int ks = 0; ks < TT / 16; ++ks) {
      const int col = ks * 16 + hg * 8;
      const bf16x8 ah = as_bf16x8(ld16(&sm.st.kh[(rb * 32 + l32) * TP + col]));
      const bf16x8 al = as_bf16x8(ld16(&sm.st.kl[(rb * 32 + l32) * TP + col]));
#pragma unroll
      for (int j = 0; j < BPW; ++j) {
        const int cb = cb0 + j;
        const bf16_t* bsrc = cb < NB ? sm.st.kt : sm.st.vt;
        const bf16x8 bo = as_bf16x8(ld16(&bsrc[((cb % NB) * 32 + l32) * TP + col]));
        acc[j] = mfma32x32x16(ah, bo, acc[j]);
        acc[j] = mfma32x32x16(al, bo, acc[j]);
      }
    }
  }
  // I + A
#pragma unroll
  for (int j = 0; j < BPW; ++j)
    if (cb0 + j == rb) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (mfma32_row(i, hg) == l32) acc[j][i] += 1.f;
    }

  // ---- blocked Gauss-Jordan.  Panels are visited as (block column cbk,
  // half PO) with cbk at run time and PO = 0, 16 compile-time; cbk runs in
  // groups whose pivot rows share one register slot OS of the factor layout
  // (rows lane + 64 OS).  Every register index and every row condition of
  // the 32 x 32 accumulator layout is then a compile-time constant.
  __syncthreads();   // the statistics tiles are dead before the union is reused
  int kpar = 0;      // panel parity: LDS buffer
  auto panel = [&](int cbk, auto osc, auto poc) __attribute__((always_inline)) {
    constexpr int OS = decltype(osc)::value;
    constexpr int PO = decltype(poc)::value;
    const int c0 = cbk * 32 + PO;
    float* pnl = sm.sv.pnl[kpar];
    float* prt = sm.sv.prt[kpar];
    kpar ^= 1;
    const bool in_panel = l32 >= PO && l32 < PO + PW;
    // (1) publish the panel columns of this wave's blocks and, from block
    // row cbk, the pivot rows (transposed; k-index kk in slot
    // (kk % 2) * 8 + kk / 2; the identity in the panel's own columns).  Then
    // preset the panel columns to the identity pattern: the update below
    // turns them into G_k.  Accumulator register i holds row
    // 8 (i / 4) + 4 hg + i % 4, so the pivot rows PO .. PO + 15 are
    // registers PO / 2 .. PO / 2 + 7 with kk = 8 (i / 4 - PO / 8) + 4 hg + i % 4.
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const int cb = cb0 + j;
      if (cb == cbk && in_panel) {
#pragma unroll
        for (int i = 0; i < 16; ++i) pnl[(rb * 32 + mfma32_row(i, hg)) * PP + (l32 - PO)] = acc[j][i];
      }
      if (rb == cbk) {
        float* dst = &prt[(cb * 32 + l32) * PP];
#pragma unroll
        for (int i = PO / 2; i < PO / 2 + 8; ++i) {
          const int kk = 8 * (i / 4 - PO / 8) + 4 * hg + (i & 3);
          const float v = (cb == cbk && in_panel) ? (l32 - PO == kk ? 1.f : 0.f) : acc[j][i];
          dst[(kk & 1) * 8 + (kk >> 1)] = v;
        }
      }
      if (cb == cbk && in_panel) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[j][i] = (rb * 32 + mfma32_row(i, hg) == cbk * 32 + l32) ? 1.f : 0.f;
      }
    }
    lds_barrier();
    // (2) factor the D x 16 panel redundantly in every wave: lane holds rows
    // lane + 64 s; pivot rows broadcast with v_readlane
    float x[RS][PW];
#pragma unroll
    for (int s2 = 0; s2 < RS; ++s2)
#pragma unroll
      for (int c4 = 0; c4 < PW / 4; ++c4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(&pnl[(lane + 64 * s2) * PP + c4 * 4]);
        x[s2][c4 * 4 + 0] = v[0];
        x[s2][c4 * 4 + 1] = v[1];
        x[s2][c4 * 4 + 2] = v[2];
        x[s2][c4 * 4 + 3] = v[3];
      }
#pragma unroll
    for (int pv = 0; pv < PW; ++pv) {
      const int ol = (c0 + pv) & 63;           // lane of the pivot row (its slot is OS)
      float rowv[PW];                          // the pivot row's panel columns (uniform)
#pragma unroll
      for (int c = 0; c < PW; ++c) rowv[c] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[OS][c]), ol));
      const float rp = 1.f / rowv[pv];
#pragma unroll
      for (int s2 = 0; s2 < RS; ++s2) {
        const float f0 = x[s2][pv] * rp;       // multiplier of this row
        // the pivot row itself: x - (1 - rp) x = rp x
        const bool own = s2 == OS && lane == ol;
        const float f = own ? 1.f - rp : f0;
#pragma unroll
        for (int c = 0; c < PW; ++c) x[s2][c] = fmaf(-f, rowv[c], x[s2][c]);
        x[s2][pv] = own ? rp : -f0;
      }
    }
    // (3) rank-16 update of this wave's blocks.  A operand: (G - I) at row
    // rb * 32 + (l % 32), k-slot 2 s + l / 32; rows of block row rb sit in
    // lane half rb % 2, slot rb / 2 of the factor layout
    float aop[PW / 2];
#pragma unroll
    for (int s2 = 0; s2 < PW / 2; ++s2) {
      const float e = RS == 1 || rb < 2 ? x[0][2 * s2] : x[RS - 1][2 * s2];
      const float o = RS == 1 || rb < 2 ? x[0][2 * s2 + 1] : x[RS - 1][2 * s2 + 1];
      float v;
      if ((rb & 1) == 0) {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(o), __float_as_uint(o), false, false);
        v = hg == 0 ? e : __uint_as_float(r[0]);
      } else {
        auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(e), __float_as_uint(e), false, false);
        v = hg == 1 ? o : __uint_as_float(r[1]);
      }
      aop[s2] = (rb * 32 + l32 == c0 + 2 * s2 + hg) ? v - 1.f : v;
    }
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
      const float* bsrc = &prt[((cb0 + j) * 32 + l32) * PP + hg * 8];
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(bsrc);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(bsrc + 4);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) acc[j] = mfma32x32x2f32(aop[s2], b0[s2], acc[j]);
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) acc[j] = mfma32x32x2f32(aop[4 + s2], b1[s2], acc[j]);
    }
  };
  for (int cbk = 0; cbk < NB / RS; ++cbk) {
    panel(cbk, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    panel(cbk, std::integral_constant<int, 0>{}, std::integral_constant<int, 16>{});
  }
  if constexpr (RS == 2)
    for (int cbk = NB / 2; cbk < NB; ++cbk) {
      panel(cbk, std::integral_constant<int, 1>{}, std::integral_constant<int, 0>{});
      panel(cbk, std::integral_constant<int, 1>{}, std::integral_constant<int, 16>{});
    }

  // ---- emit: T = X diag(alpha), U = X W (video frame) or S_text = X W (text
  // frame); X itself when Xf is set (the backward pass solves with it)
  const size_t DD = (size_t)D * D;
  const float* al = alpha_row(a, bh, fr);
  float* Xo = a.Xf ? a.Xf + ((size_t)bh * (g.F + 1) + fr) * DD : nullptr;
#pragma unroll
  for (int j = 0; j < BPW; ++j) {
    const int cb = cb0 + j;
    const int col = (cb % NB) * 32 + l32;
    if (cb < NB) {
      const float aj = text ? 1.f : al[col];
      float* Tout = text ? nullptr : a.Tf + ((size_t)bh * g.F + fr) * DD;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const size_t e = (size_t)(rb * 32 + mfma32_row(i, hg)) * D + col;
        if (Xo) Xo[e] = acc[j][i];
        if (!text) Tout[e] = acc[j][i] * aj;
      }
    } else {
      float* Uout = text ? a.S_text + (size_t)bh * DD : a.Uf + ((size_t)bh * g.F + fr) * DD;
#pragma unroll
      for (int i = 0; i < 16; ++i) Uout[(size_t)(rb * 32 + mfma32_row(i, hg)) * D + col] = acc[j][i];
    }
  }
}

template <typename T>
hipError_t launch_vda_frame_solve(const Geometry& g, const T* k, const T* v, const float* beta,
                                  const float* alpha, const T* k_text, const T* v_text,
                                  const float* beta_text, float* Tf, float* Uf, float* S_text,
                                  hipStream_t s, float* Xf) {
  SolveArgs<T> a{g, k, v, beta, alpha, k_text, v_text, beta_text, Tf, Uf, S_text, Xf};
  const unsigned grid = (unsigned)(g.B * g.H * (g.F + 1));
  switch (g.D) {
    case 16: vda_frame_solve_kernel<T, 16><<<grid, 256, 0, s>>>(a); break;
    case 32: vda_frame_solve_kernel<T, 32><<<grid, 256, 0, s>>>(a); break;
    case 64: vda_frame_solve_kernel<T, 64><<<grid, 256, 0, s>>>(a); break;
    case 128: vda_frame_solve_kernel<T, 128><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <>
hipError_t launch_vda_frame_solve<bf16_t>(const Geometry& g, const bf16_t* k, const bf16_t* v,
                                          const float* beta, const float* alpha,
                                          const bf16_t* k_text, const bf16_t* v_text,
                                          const float* beta_text, float* Tf, float* Uf,
                                          float* S_text, hipStream_t s, float* Xf) {
  SolveArgs<bf16_t> a{g, k, v, beta, alpha, k_text, v_text, beta_text, Tf, Uf, S_text, Xf};
  const unsigned grid = (unsigned)(g.B * g.H * (g.F + 1));
  switch (g.D) {
    case 16: vda_frame_solve_kernel<bf16_t, 16><<<grid, 256, 0, s>>>(a); break;
    case 32: vda_frame_solve_kernel<bf16_t, 32><<<grid, 256, 0, s>>>(a); break;
    case 64: vda_frame_solve_mfma_kernel<64><<<grid, 256, 0, s>>>(a); break;
    case 128: vda_frame_solve_mfma_kernel<128><<<grid, 256, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_vda_frame_solve<float>(const Geometry&, const float*, const float*,
                                                  const float*, const float*, const float*,
                                                  const float*, const float*, float*, float*,
                                                  float*, hipStream_t, float*);

}  // namespace vdn
