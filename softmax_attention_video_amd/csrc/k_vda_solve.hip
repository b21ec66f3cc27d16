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
// Our design: one workgroup (256 threads, a 16 x 16 thread grid) per
// (b, h, frame), frame index F being the text frame.  Thread (tr, tc) owns
// rows tr*R..tr*R+R-1 of the augmented matrix [I + A | W] in columns
// tc*R..tc*R+R-1 of each half (R = D / 16), i.e. 2 R^2 fp32 registers.
// I + A is symmetric positive definite (eigenvalues >= 1), so the
// elimination needs no pivoting; each pivot step broadcasts the pivot row
// and column through double-buffered LDS with one barrier.
//
// Statistics: the bf16 kernel (D = 64, 128) contracts over tokens on
// v_mfma_f32_32x32x16_bf16.  Tokens must be the contracted (lane-contiguous)
// index, so each 64-token tile is transposed into LDS ([channel][token]).
// beta * K is formed in fp32 and split into bf16 hi + lo parts, so A and W
// carry ~16 more mantissa bits than a single bf16 product.  The generic
// kernel (fp32 storage, any D) accumulates in fp32 on the VALU.
#include "vdn_common.h"
#include "vdn_internal.h"

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
// bf16 kernel: MFMA statistics (D = 64, 128).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void vda_frame_solve_mfma_kernel(SolveArgs<bf16_t> a) {
  constexpr int R = D / 16;
  constexpr int TT = 64;            // tokens per tile
  constexpr int TP = TT + 8;        // transposed tile pitch (bf16)
  constexpr int NB = D / 32;        // 32-blocks per matrix side
  constexpr int BPW = 2 * NB * NB / 4;   // output blocks per wave (A and W)
  constexpr int XP = D + 1;         // fp32 transfer pitch
  constexpr int PAIRS = TT / 2 * (D / 8) / 256;   // (token pair, 8-channel chunk) per thread
  struct StatsTiles {
    bf16_t kt[D * TP];    // K^T
    bf16_t kh[D * TP];    // (beta K)^T, bf16 high part
    bf16_t kl[D * TP];    // (beta K)^T, bf16 low part
    bf16_t vt[D * TP];    // V^T
  };
  union Smem {
    StatsTiles st;
    float xfer[D * XP];
  };
  __shared__ __attribute__((aligned(16))) Smem sm;
  __shared__ GJShared sh;

  const Geometry& g = a.g;
  const int fr = blockIdx.x % (g.F + 1);
  const int bh = blockIdx.x / (g.F + 1);
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
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

  if (ntok > 0) fetch(0);
  for (long long t0 = 0; t0 < ntok; t0 += TT) {
    __syncthreads();
    stage();
    __syncthreads();
    if (t0 + TT < ntok) fetch(t0 + TT);
#pragma unroll
    for (int ks = 0; ks < TT / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < BPW; ++i) {
        const int bi = wave * BPW + i;
        const bool wblk = bi >= NB * NB;                 // block of W (else of A)
        const int mb = (bi % (NB * NB)) / NB, nb = bi % NB;
        const int col = ks * 16 + hg * 8;
        const bf16x8 ah = as_bf16x8(ld16(&sm.st.kh[(mb * 32 + l32) * TP + col]));
        const bf16x8 al = as_bf16x8(ld16(&sm.st.kl[(mb * 32 + l32) * TP + col]));
        const bf16_t* bsrc = wblk ? sm.st.vt : sm.st.kt;
        const bf16x8 bo = as_bf16x8(ld16(&bsrc[(nb * 32 + l32) * TP + col]));
        acc[i] = mfma32x32x16(ah, bo, acc[i]);
        acc[i] = mfma32x32x16(al, bo, acc[i]);
      }
    }
  }

  // accumulators -> GJ ownership, A first then W, through one fp32 buffer
  float m[R][R], w[R][R];
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      const int bi = wave * BPW + i;
      if ((bi >= NB * NB) != (pass == 1)) continue;
      const int mb = (bi % (NB * NB)) / NB, nb = bi % NB;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        sm.xfer[(mb * 32 + mfma32_row(r, hg)) * XP + nb * 32 + l32] = acc[i][r];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float x = sm.xfer[(tr * R + i) * XP + tc * R + j];
        if (pass == 0) m[i][j] = x; else w[i][j] = x;
      }
  }
  if (tr == tc) {
#pragma unroll
    for (int i = 0; i < R; ++i) m[i][i] += 1.f;
  }
  gauss_jordan<D>(m, w, sh, tr, tc);
  emit_solution<D>(g, a.alpha, a.Tf, a.Uf, a.S_text, a.Xf, bh, fr, text, m, w, tr, tc);
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
