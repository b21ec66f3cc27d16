// Backward pass of the window + boundary-anchor Softmax branch.
//
// Paper ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream
// Video Generation"), method, local Softmax window and branch calibration,
// defines the forward Ohat_s = g_s * softmax(scale q k^T) v over the visible
// keys; the experiments train through it.  The gradients are the chain rule
// of that definition: with dO = g_s * dOhat and Dq = rowsum(dO * O_s),
//   P = exp(scale q.k - lse),   dP = dO . v,   dS = P (dP - Dq),
//   dQ = scale sum_keys dS k,   dK = scale sum_queries dS q,
//   dV = sum_queries P dO,      dg_s = rowsum(dOhat * O_s),
// where lse is the forward's log-sum-exp, so P needs no renormalisation.
//
// Work split: a query-stationary pass computes dQ over the same items as the
// forward (query groups and their key spans); a key-stationary pass computes
// dK and dV.  Visibility is symmetric, so the forward's items read with the
// roles swapped (the group's frames as keys, its spans as the queries that
// see them) cover every (query, key) pair exactly once, and every output row
// is written by one workgroup: no atomics.
#include "vdn_common.h"
#include "vdn_internal.h"
#include "window_items.h"

#include <math.h>

namespace vdn {

// ---------------------------------------------------------------------------
// Preprocess: dO (head-major) = g * dOhat, Dq = g * rowsum(dOhat * O),
// dg = rowsum(dOhat * O).  dOhat and O in the output layout [B,L,H,D].
// One thread per 8 channels of a (b, l, h) row; a row's D/8 lanes reduce
// with shuffles.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void softmax_bwd_prep_kernel(Geometry g, const T* __restrict__ o,
                                                               const T* __restrict__ dout,
                                                               const float* __restrict__ g_s,
                                                               T* __restrict__ do_hm,
                                                               float* __restrict__ Dq,
                                                               float* __restrict__ dg) {
  const int D = g.D, cpr = D / 8;                          // lanes per row (2..16)
  const long long rows = (long long)g.B * g.L * g.H;       // in output order (b, l, h)
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = gid / cpr;
  const int c8 = (int)(gid % cpr);
  const bool live = row < rows;
  const long long r = live ? row : 0;
  const int h = (int)(r % g.H);
  const long long bl = r / g.H;                            // b * L + l
  const long long b = bl / g.L, l = bl % g.L;
  const size_t src = (size_t)r * D + c8 * 8;
  float x[8], y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = live ? Elem<T>::load(dout, src + j) : 0.f;
    y[j] = live ? Elem<T>::load(o, src + j) : 0.f;
  }
  float part = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) part = fmaf(x[j], y[j], part);
  for (int off = 1; off < cpr; off <<= 1) part += __shfl_xor(part, off);
  if (!live) return;
  const size_t hrow = ((size_t)b * g.H + h) * g.L + l;     // head-major row
  const float gate = g_s ? g_s[hrow] : 1.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) Elem<T>::store(do_hm, hrow * D + c8 * 8 + j, gate * x[j]);
  if (c8 == 0) {
    Dq[hrow] = gate * part;
    if (dg) dg[hrow] = part;
  }
}

template <typename T>
hipError_t launch_softmax_bwd_prep(const Geometry& g, const T* o, const T* dout, const float* g_s,
                                   T* do_hm, float* Dq, float* dg, hipStream_t s) {
  const long long n = (long long)g.B * g.L * g.H * (g.D / 8);
  if (n == 0) return hipSuccess;
  softmax_bwd_prep_kernel<T><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(g, o, dout, g_s, do_hm, Dq, dg);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Generic SIMT kernels (fp32 or bf16 storage, any D <= 128, any N).
// dQ: one thread per query, key tiles of 32 staged through LDS.
// ---------------------------------------------------------------------------
template <typename T, int DMAX>
__global__ __launch_bounds__(128) void softmax_bwd_dq_simt_kernel(
    Geometry g, SoftmaxWork w, const T* __restrict__ qp, const T* __restrict__ kp,
    const T* __restrict__ vp, const T* __restrict__ dop, const float* __restrict__ lse,
    const float* __restrict__ Dq, T* __restrict__ dq, float scale) {
  constexpr int BQ = 128, BK = 32;
  __shared__ float Ks[BK][DMAX + 1];
  __shared__ float Vs[BK][DMAX + 1];
  Item it;
  int q0;
  if (!decode_item<false>(g, w, BQ, blockIdx.x, 0, it, q0)) return;
  const int D = g.D;
  const long long L = g.L;
  const int qrow = q0 + threadIdx.x;
  const bool qvalid = qrow < it.q_end;
  const size_t base = (size_t)it.bh * L * D;
  float qv[DMAX], dov[DMAX], acc[DMAX];
#pragma unroll
  for (int j = 0; j < DMAX; ++j) {
    qv[j] = (j < D && qvalid) ? Elem<T>::load(qp, base + (size_t)qrow * D + j) : 0.f;
    dov[j] = (j < D && qvalid) ? Elem<T>::load(dop, base + (size_t)qrow * D + j) : 0.f;
    acc[j] = 0.f;
  }
  const float lq = qvalid ? lse[(size_t)it.bh * L + qrow] : 0.f;
  const float dq_ = qvalid ? Dq[(size_t)it.bh * L + qrow] : 0.f;
  const SpanWalk<BK, 3> walk(it);
  for (int jt = 0; jt < walk.n; ++jt) {
    int ks, nk;
    walk.tile(jt, ks, nk);
    __syncthreads();
    for (int e = threadIdx.x; e < BK * D; e += blockDim.x) {
      const int r = e / D, c = e % D;
      Ks[r][c] = r < nk ? Elem<T>::load(kp, base + (size_t)(ks + r) * D + c) : 0.f;
      Vs[r][c] = r < nk ? Elem<T>::load(vp, base + (size_t)(ks + r) * D + c) : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < nk; ++r) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int j = 0; j < DMAX; ++j)
        if (j < D) {
          s = fmaf(qv[j], Ks[r][j], s);
          dp = fmaf(dov[j], Vs[r][j], dp);
        }
      const float p = expf(fmaf(s, scale, -lq));
      const float ds = p * (dp - dq_);
#pragma unroll
      for (int j = 0; j < DMAX; ++j)
        if (j < D) acc[j] = fmaf(ds, Ks[r][j], acc[j]);
    }
  }
  if (!qvalid) return;
#pragma unroll
  for (int j = 0; j < DMAX; ++j)
    if (j < D) Elem<T>::store(dq, base + (size_t)qrow * D + j, acc[j] * scale);
}

// dK, dV: one thread per key (the item's frames read as key frames, its
// spans as the query frames that see them), query tiles of 32 with their
// lse and Dq staged through LDS.
template <typename T, int DMAX>
__global__ __launch_bounds__(128) void softmax_bwd_dkdv_simt_kernel(
    Geometry g, SoftmaxWork w, const T* __restrict__ qp, const T* __restrict__ kp,
    const T* __restrict__ vp, const T* __restrict__ dop, const float* __restrict__ lse,
    const float* __restrict__ Dq, T* __restrict__ dk, T* __restrict__ dv, float scale) {
  constexpr int BK = 128, BQ = 32;
  __shared__ float Qs[BQ][DMAX + 1];
  __shared__ float Ds[BQ][DMAX + 1];
  __shared__ float Ls[BQ], Dd[BQ];
  Item it;
  int k0;
  if (!decode_item<false>(g, w, BK, blockIdx.x, 0, it, k0)) return;
  const int D = g.D;
  const long long L = g.L;
  const int krow = k0 + threadIdx.x;
  const bool kvalid = krow < it.q_end;
  const size_t base = (size_t)it.bh * L * D;
  float kv[DMAX], vv[DMAX], ak[DMAX], av[DMAX];
#pragma unroll
  for (int j = 0; j < DMAX; ++j) {
    kv[j] = (j < D && kvalid) ? Elem<T>::load(kp, base + (size_t)krow * D + j) : 0.f;
    vv[j] = (j < D && kvalid) ? Elem<T>::load(vp, base + (size_t)krow * D + j) : 0.f;
    ak[j] = 0.f;
    av[j] = 0.f;
  }
  const SpanWalk<BQ, 3> walk(it);
  for (int jt = 0; jt < walk.n; ++jt) {
    int qs, nq;
    walk.tile(jt, qs, nq);
    __syncthreads();
    for (int e = threadIdx.x; e < BQ * D; e += blockDim.x) {
      const int r = e / D, c = e % D;
      Qs[r][c] = r < nq ? Elem<T>::load(qp, base + (size_t)(qs + r) * D + c) : 0.f;
      Ds[r][c] = r < nq ? Elem<T>::load(dop, base + (size_t)(qs + r) * D + c) : 0.f;
    }
    if (threadIdx.x < BQ) {
      const int r = threadIdx.x;
      Ls[r] = r < nq ? lse[(size_t)it.bh * L + qs + r] : 0.f;
      Dd[r] = r < nq ? Dq[(size_t)it.bh * L + qs + r] : 0.f;
    }
    __syncthreads();
    for (int r = 0; r < nq; ++r) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int j = 0; j < DMAX; ++j)
        if (j < D) {
          s = fmaf(Qs[r][j], kv[j], s);
          dp = fmaf(Ds[r][j], vv[j], dp);
        }
      const float p = expf(fmaf(s, scale, -Ls[r]));
      const float ds = p * (dp - Dd[r]);
#pragma unroll
      for (int j = 0; j < DMAX; ++j)
        if (j < D) {
          av[j] = fmaf(p, Ds[r][j], av[j]);
          ak[j] = fmaf(ds, Qs[r][j], ak[j]);
        }
    }
  }
  if (!kvalid) return;
#pragma unroll
  for (int j = 0; j < DMAX; ++j)
    if (j < D) {
      Elem<T>::store(dk, base + (size_t)krow * D + j, ak[j] * scale);
      Elem<T>::store(dv, base + (size_t)krow * D + j, av[j]);
    }
}

template <typename T>
hipError_t launch_softmax_bwd_simt(const Geometry& g, const T* q, const T* k, const T* v,
                                   const T* do_hm, const float* lse, const float* Dq, T* dq, T* dk,
                                   T* dv, float scale, hipStream_t s) {
  const SoftmaxWork wq = window_work(g, 128);
  const SoftmaxWork wk = window_work(g, 128);
  if (wq.grid == 0) return hipSuccess;
#define VDN_BWD_SIMT(DM)                                                                           \
  softmax_bwd_dq_simt_kernel<T, DM><<<wq.grid, 128, 0, s>>>(g, wq, q, k, v, do_hm, lse, Dq, dq, scale); \
  softmax_bwd_dkdv_simt_kernel<T, DM><<<wk.grid, 128, 0, s>>>(g, wk, q, k, v, do_hm, lse, Dq, dk, dv, scale)
  if (g.D <= 16) {
    VDN_BWD_SIMT(16);
  } else if (g.D <= 32) {
    VDN_BWD_SIMT(32);
  } else if (g.D <= 64) {
    VDN_BWD_SIMT(64);
  } else {
    VDN_BWD_SIMT(128);
  }
#undef VDN_BWD_SIMT
  return hipGetLastError();
}

template hipError_t launch_softmax_bwd_prep<float>(const Geometry&, const float*, const float*,
                                                   const float*, float*, float*, float*, hipStream_t);
template hipError_t launch_softmax_bwd_prep<bf16_t>(const Geometry&, const bf16_t*, const bf16_t*,
                                                    const float*, bf16_t*, float*, float*,
                                                    hipStream_t);
template hipError_t launch_softmax_bwd_simt<float>(const Geometry&, const float*, const float*,
                                                   const float*, const float*, const float*,
                                                   const float*, float*, float*, float*, float,
                                                   hipStream_t);
template hipError_t launch_softmax_bwd_simt<bf16_t>(const Geometry&, const bf16_t*, const bf16_t*,
                                                    const bf16_t*, const bf16_t*, const float*,
                                                    const float*, bf16_t*, bf16_t*, bf16_t*, float,
                                                    hipStream_t);

}  // namespace vdn
