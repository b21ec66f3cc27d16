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
// tc*R..tc*R+R-1 of each half (R = D / 16), i.e. 2 R^2 fp32 registers.  The
// statistics are accumulated straight into that ownership, so A and W never
// leave registers.  I + A is symmetric positive definite (eigenvalues >= 1),
// so the elimination needs no pivoting; each pivot step broadcasts the pivot
// row and column through double-buffered LDS with one barrier.
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
};

template <typename T, int D>
__global__ __launch_bounds__(256) void vda_frame_solve_kernel(SolveArgs<T> a) {
  constexpr int R = D / 16;
  constexpr int TT = 32;  // tokens per LDS stage
  __shared__ float Ks[TT][D + 1];
  __shared__ float Vs[TT][D + 1];
  __shared__ float Bs[TT];
  __shared__ float colbuf[2][D];
  __shared__ float rowM[2][D];
  __shared__ float rowW[2][D];

  const Geometry& g = a.g;
  const int fr = blockIdx.x % (g.F + 1);
  const int bh = blockIdx.x / (g.F + 1);
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  const bool text = (fr == g.F);
  const size_t DD = (size_t)D * D;

  if (!text && g.anchors && (fr == 0 || fr == g.F - 1)) {
    // Anchor frames are excluded from both scans: decay only.
    const float* al = a.alpha + ((size_t)bh * g.F + fr) * D;
    float* Tout = a.Tf + ((size_t)bh * g.F + fr) * DD;
    float* Uout = a.Uf + ((size_t)bh * g.F + fr) * DD;
    for (int e = tid; e < D * D; e += 256) {
      const int i = e / D, j = e % D;
      Tout[e] = (i == j) ? al[j] : 0.f;
      Uout[e] = 0.f;
    }
    return;
  }

  const T* kp;
  const T* vp;
  const float* bp;
  long long ntok;
  if (text) {
    ntok = g.T;
    kp = a.k_text + (size_t)bh * g.T * D;
    vp = a.v_text + (size_t)bh * g.T * D;
    bp = a.beta_text + (size_t)bh * g.T;
  } else {
    ntok = g.N;
    const size_t off = (size_t)bh * g.L + (size_t)fr * g.N;
    kp = a.k + off * D;
    vp = a.v + off * D;
    bp = a.beta + off;
  }

  float m[R][R], w[R][R];
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = 0; j < R; ++j) {
      m[i][j] = 0.f;
      w[i][j] = 0.f;
    }

  // ---- statistics: m += beta k k^T, w += beta k v^T over the tokens ----
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

  // ---- in-place Gauss-Jordan on [I + A | W] -> [(I + A)^{-1} | (I + A)^{-1} W] ----
  for (int kb = 0; kb < 16; ++kb) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int k = kb * R + r;
      const int buf = k & 1;
      if (tc == kb) {
#pragma unroll
        for (int i = 0; i < R; ++i) colbuf[buf][tr * R + i] = m[i][r];
      }
      if (tr == kb) {
#pragma unroll
        for (int j = 0; j < R; ++j) {
          rowM[buf][tc * R + j] = m[r][j];
          rowW[buf][tc * R + j] = w[r][j];
        }
      }
      __syncthreads();
      const float p = 1.f / rowM[buf][k];
      float cik[R], rkj[R], rkw[R];
#pragma unroll
      for (int i = 0; i < R; ++i) cik[i] = colbuf[buf][tr * R + i] * p;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        rkj[j] = rowM[buf][tc * R + j];
        rkw[j] = rowW[buf][tc * R + j];
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

  // ---- emit T = X diag(alpha), U = X W (or S_text) ----
  if (text) {
    float* S = a.S_text + (size_t)bh * DD;
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int j = 0; j < R; ++j) S[(size_t)(tr * R + i) * D + tc * R + j] = w[i][j];
    return;
  }
  const float* al = a.alpha + ((size_t)bh * g.F + fr) * D;
  float* Tout = a.Tf + ((size_t)bh * g.F + fr) * DD;
  float* Uout = a.Uf + ((size_t)bh * g.F + fr) * DD;
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
hipError_t launch_vda_frame_solve(const Geometry& g, const T* k, const T* v, const float* beta,
                                  const float* alpha, const T* k_text, const T* v_text,
                                  const float* beta_text, float* Tf, float* Uf, float* S_text,
                                  hipStream_t s) {
  SolveArgs<T> a{g, k, v, beta, alpha, k_text, v_text, beta_text, Tf, Uf, S_text};
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

template hipError_t launch_vda_frame_solve<float>(const Geometry&, const float*, const float*,
                                                  const float*, const float*, const float*,
                                                  const float*, const float*, float*, float*,
                                                  float*, hipStream_t);
template hipError_t launch_vda_frame_solve<bf16_t>(const Geometry&, const bf16_t*, const bf16_t*,
                                                   const float*, const float*, const bf16_t*,
                                                   const bf16_t*, const float*, float*, float*,
                                                   float*, hipStream_t);

}  // namespace vdn
