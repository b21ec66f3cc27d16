// Backward pass of the linear (VDA) branch.
//
// Paper ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream
// Video Generation"): the Video Delta Attention section defines the frame
// statistics A_f = K_f^T B_f K_f, W_f = K_f^T B_f V_f and the frame update
// S_f = (I + A_f)^{-1} (diag(alpha_f) S_{f-1} + W_f); the method's
// bidirectional linear attention reads each query frame's memory at chunk
// boundaries through a decay bridge, M_t = diag(D_fwd) P_fwd[i_f] +
// diag(D_rev) P_rev[i_r], and sums the two readouts; branch calibration
// RMS-normalises the readout and gates it.  The experiments train through
// this operator; its gradients are the chain rule of those definitions.
//
// With X_f = (I + A_f)^{-1} (symmetric) and lambda_f the adjoint of the
// state after frame f, one frame of either scan gives
//   Z_f = X_f lambda_f,  dW_f += Z_f,  dA_f -= Z_f S_f^T,
//   dalpha_f += rowsum(Z_f * S_prev),  lambda_prev = diag(alpha_f) Z_f,
// and an anchor frame (decay only) the same with Z_f = lambda_f and no
// dA/dW.  The statistics then give, per token, with dA_sym = dA + dA^T:
//   dk = beta (k dA_sym + v dW^T),  dv = beta k dW,
//   dbeta = 1/2 (k dA_sym) . k + (k dW) . v.
//
// Our organisation follows the forward's chunk structure instead of running
// one long sequential adjoint per head:
//   1. readout backward, one workgroup per (b, h, query frame): recompute
//      O = q M_t, the RMSNorm/gate adjoint, dq = dO M_t^T, G_t = Q_t^T dO_t,
//      and the bridge adjoints dD = rowsum(G_t * P);
//   2. dP[i] = sum over the query frames reading slot i of diag(D_t) G_t;
//   3. the bridges' alpha gradients, per (b, h) and channel, as a two-pass
//      running product (no division by alpha);
//   4. the chunk-level adjoint scan mu[i] = dP[i] + T_c^T mu[i +- 1] with
//      the composed chunk maps T_c of the forward (sequential over chunks);
//   5. the text state's adjoint, Z_text = X_text * s (mu_fwd[0] + mu_rev[C]);
//   6. per (b, h, direction, chunk): recompute the chunk's frame states from
//      its boundary state, then the frame adjoints Z_f from the chunk's end
//      adjoint -- the chunks run in parallel;
//   7. per (b, h, frame): dA_sym and dW from Z and the states, the scan's
//      alpha term, and the token gradients.
// All small-matrix work is fp32.  State-sized products act column by column,
// so kernels 4-6 split the d_v columns into 32-wide blocks.
#include "vdn_common.h"
#include "vdn_internal.h"

namespace vdn {

namespace {

constexpr int kBCB = 32;   // state columns per workgroup in the chain kernels

template <typename T>
struct VdaBwdArgs {
  Geometry g;
  const T* q;
  const T* k;
  const T* v;
  const float* beta;
  const float* alpha;
  const T* k_text;
  const T* v_text;
  const float* beta_text;
  const float* g_l;
  const float* gamma;
  const T* d_out;        // [B, L, H, D]
  float eps;
  float init_scale;
  const float* Pf;       // [BH, C+1, DD]
  const float* Pr;
  const float* St;       // [BH, DD]
  const float* Xf;       // [BH, F+1, DD]
  const float* Tc;       // [BH, 2, C, DD]
  float* G;              // [BH, F, DD]
  float* Dbr;            // [BH, 2, F, D] bridge products
  float* dDbr;           // [BH, 2, F, D] their adjoints
  float* dgp;            // [BH, F, D] dgamma partial sums (nullable)
  float* dP;             // [BH, 2, C+1, DD]
  float* mu;             // [BH, 2, C+1, DD]
  float* Sst;            // [BH, 2, F+1, DD] frame states
  float* Zst;            // [BH, 2, F, DD]
  float* ZT;             // [BH, DD]
  float* Rscr;           // [BH, F, D]
  T* dq;
  T* dk;
  T* dv;
  float* dbeta;
  float* dalpha;
  T* dk_text;
  T* dv_text;
  float* dbeta_text;
  float* dg_l;           // nullable
};

__device__ __forceinline__ bool is_anchor_frame(const Geometry& g, int f) {
  return g.anchors && (f == 0 || f == g.F - 1);
}

// Sum over the 16 lanes of a lane group (lanes 16m .. 16m+15).
__device__ __forceinline__ float sum16(float x) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m, 16);
  return x;
}

__device__ __forceinline__ float sum64(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

// ---------------------------------------------------------------------------
// 1. Readout backward.  One workgroup (256 threads) per (b, h, query frame).
//    Thread (grp, sub) handles token grp of a 16-token tile and the columns
//    sub + 16 j; for G = Q^T dO it owns rows tr + 16 i, columns tc + 16 j
//    (tr = grp, tc = sub).  M_t lives in LDS with pitch D + 1, so the row
//    reads of q M and the column reads of dO M^T are both conflict-free.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void vda_bwd_readout_kernel(VdaBwdArgs<T> a) {
  constexpr int CPT = D / 16, TOK = 16, MP = D + 1;
  __shared__ float Ms[D * MP];
  __shared__ float Qs[TOK][MP];
  __shared__ float Os[TOK][MP];
  __shared__ float dfs[D], drs[D];

  const Geometry& g = a.g;
  const int t = blockIdx.x % g.F;
  const int bh = blockIdx.x / g.F;
  const int tid = threadIdx.x, grp = tid >> 4, sub = tid & 15;
  const size_t DD = (size_t)D * D;
  int i_f, ws, i_r, we;
  readout_indices(g, t, i_f, ws, i_r, we);
  const float* al = a.alpha + (size_t)bh * g.F * D;
  for (int c = tid; c < D; c += 256) {
    float df = 1.f, dr = 1.f;
    for (int f = ws; f <= t; ++f) df *= al[(size_t)f * D + c];
    for (int f = t; f <= we; ++f) dr *= al[(size_t)f * D + c];
    dfs[c] = df;
    drs[c] = dr;
    a.Dbr[(((size_t)bh * 2 + 0) * g.F + t) * D + c] = df;
    a.Dbr[(((size_t)bh * 2 + 1) * g.F + t) * D + c] = dr;
  }
  __syncthreads();
  const float* pf = a.Pf + ((size_t)bh * (g.C + 1) + i_f) * DD;
  const float* pr = a.Pr + ((size_t)bh * (g.C + 1) + i_r) * DD;
  for (int e = tid; e < D * D; e += 256) {
    const int r = e / D, c = e % D;
    Ms[r * MP + c] = dfs[r] * pf[e] + drs[r] * pr[e];
  }
  float gm[CPT], gacc[CPT], Gacc[CPT][CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    gm[j] = a.gamma ? a.gamma[sub + 16 * j] : 1.f;
    gacc[j] = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) Gacc[i][j] = 0.f;
  }
  const int bidx = bh / g.H, h = bh % g.H;
  const size_t tok0 = (size_t)bh * g.L + (size_t)t * g.N;
  for (int n0 = 0; n0 < g.N; n0 += TOK) {
    __syncthreads();
    for (int e = tid; e < TOK * D; e += 256) {
      const int r = e / D, c = e % D;
      Qs[r][c] = (n0 + r < g.N) ? Elem<T>::load(a.q, (tok0 + n0 + r) * D + c) : 0.f;
    }
    __syncthreads();
    float o[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) o[j] = 0.f;
    for (int kk = 0; kk < D; ++kk) {
      const float qk = Qs[grp][kk];
#pragma unroll
      for (int j = 0; j < CPT; ++j) o[j] = fmaf(qk, Ms[kk * MP + sub + 16 * j], o[j]);
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) ss = fmaf(o[j], o[j], ss);
    ss = sum16(ss);
    const int n = n0 + grp;
    const bool valid = n < g.N;
    const size_t l = (size_t)t * g.N + n;
    const float inv = rsqrtf(ss / (float)D + a.eps);
    const float gate = valid ? a.g_l[(size_t)bh * g.L + l] : 0.f;
    const size_t ob = (((size_t)bidx * g.L + l) * g.H + h) * D;
    float u[CPT], y[CPT], dgv = 0.f, uy = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const float dOh = valid ? Elem<T>::load(a.d_out, ob + sub + 16 * j) : 0.f;
      y[j] = valid ? o[j] * inv : 0.f;     // padded rows: o = 0, and inv = inf when eps = 0
      u[j] = gate * gm[j] * dOh;
      dgv = fmaf(dOh * gm[j], y[j], dgv);
      uy = fmaf(u[j], y[j], uy);
      gacc[j] = fmaf(dOh * gate, y[j], gacc[j]);
    }
    dgv = sum16(dgv);
    uy = sum16(uy);
    if (valid && sub == 0 && a.dg_l) a.dg_l[(size_t)bh * g.L + l] = dgv;
    const float muy = uy / (float)D;
#pragma unroll
    for (int j = 0; j < CPT; ++j) Os[grp][sub + 16 * j] = valid ? inv * (u[j] - y[j] * muy) : 0.f;
    __syncthreads();
    // dq = dO M^T
    float dqv[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) dqv[j] = 0.f;
    for (int vv = 0; vv < D; ++vv) {
      const float dov = Os[grp][vv];
#pragma unroll
      for (int j = 0; j < CPT; ++j) dqv[j] = fmaf(dov, Ms[(sub + 16 * j) * MP + vv], dqv[j]);
    }
    if (valid) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) Elem<T>::store(a.dq, (tok0 + n) * D + sub + 16 * j, dqv[j]);
    }
    // G += Q^T dO over the tile
    for (int nn = 0; nn < TOK; ++nn) {
      float qv[CPT], dv_[CPT];
#pragma unroll
      for (int i = 0; i < CPT; ++i) qv[i] = Qs[nn][grp + 16 * i];
#pragma unroll
      for (int j = 0; j < CPT; ++j) dv_[j] = Os[nn][sub + 16 * j];
#pragma unroll
      for (int i = 0; i < CPT; ++i)
#pragma unroll
        for (int j = 0; j < CPT; ++j) Gacc[i][j] = fmaf(qv[i], dv_[j], Gacc[i][j]);
    }
  }
  // G_t, and the bridge adjoints dD = rowsum(G * P)
  float* Go = a.G + ((size_t)bh * g.F + t) * DD;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int r = grp + 16 * i;
    float sf = 0.f, sr = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = sub + 16 * j;
      Go[(size_t)r * D + c] = Gacc[i][j];
      sf = fmaf(Gacc[i][j], pf[(size_t)r * D + c], sf);
      sr = fmaf(Gacc[i][j], pr[(size_t)r * D + c], sr);
    }
    sf = sum16(sf);
    sr = sum16(sr);
    if (sub == 0) {
      a.dDbr[(((size_t)bh * 2 + 0) * g.F + t) * D + r] = sf;
      a.dDbr[(((size_t)bh * 2 + 1) * g.F + t) * D + r] = sr;
    }
  }
  if (a.dgp) {
    __syncthreads();
#pragma unroll
    for (int j = 0; j < CPT; ++j) Qs[grp][sub + 16 * j] = gacc[j];
    __syncthreads();
    for (int c = tid; c < D; c += 256) {
      float s = 0.f;
      for (int r = 0; r < TOK; ++r) s += Qs[r][c];
      a.dgp[((size_t)bh * g.F + t) * D + c] = s;
    }
  }
}

// ---------------------------------------------------------------------------
// 2. dP[dir][i] = sum_{t reading slot i} diag(D_dir[t]) G_t.
//    One workgroup per (b, h, direction, slot).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void vda_bwd_dp_kernel(VdaBwdArgs<T> a) {
  constexpr int PER = D * D / 256 > 0 ? D * D / 256 : 1;
  const Geometry& g = a.g;
  int id = blockIdx.x;
  const int slot = id % (g.C + 1); id /= (g.C + 1);
  const int dir = id % 2;
  const int bh = id / 2;
  const size_t DD = (size_t)D * D;
  float acc[PER];
#pragma unroll
  for (int m = 0; m < PER; ++m) acc[m] = 0.f;
  for (int t = 0; t < g.F; ++t) {
    int i_f, ws, i_r, we;
    readout_indices(g, t, i_f, ws, i_r, we);
    if ((dir == 0 ? i_f : i_r) != slot) continue;
    const float* Gt = a.G + ((size_t)bh * g.F + t) * DD;
    const float* sc = a.Dbr + (((size_t)bh * 2 + dir) * g.F + t) * D;
#pragma unroll
    for (int m = 0; m < PER; ++m) {
      const int e = threadIdx.x + 256 * m;
      if (e < D * D) acc[m] = fmaf(sc[e / D], Gt[e], acc[m]);
    }
  }
  float* out = a.dP + (((size_t)bh * 2 + dir) * (g.C + 1) + slot) * DD;
#pragma unroll
  for (int m = 0; m < PER; ++m) {
    const int e = threadIdx.x + 256 * m;
    if (e < D * D) out[e] = acc[m];
  }
}

// ---------------------------------------------------------------------------
// 3. Bridge alpha gradients.  D_fwd[t] = prod_{f=ws..t} alpha_f: the queries
//    sharing a bridge start a (one group) contribute to alpha_f, f >= a,
//      pre(f) * R(f),  pre(f) = prod_{a..f-1} alpha,
//      R(f) = [f in group] dD_f + alpha_{f+1} R(f+1)   (f up to the group's last query);
//    the reverse bridges t..we mirror this.  One thread per channel; R is
//    kept in a per-thread column of Rscr.  Writes (initialises) dalpha.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(128) void vda_bwd_alpha_bridge_kernel(VdaBwdArgs<T> a) {
  const Geometry& g = a.g;
  const int bh = blockIdx.x;
  const int c = threadIdx.x;
  if (c >= D) return;
  const float* al = a.alpha + (size_t)bh * g.F * D + c;
  float* da = a.dalpha + (size_t)bh * g.F * D + c;
  float* R = a.Rscr + (size_t)bh * g.F * D + c;
  const float* dDf = a.dDbr + ((size_t)bh * 2 + 0) * g.F * D + c;
  const float* dDr = a.dDbr + ((size_t)bh * 2 + 1) * g.F * D + c;
  for (int f = 0; f < g.F; ++f) da[(size_t)f * D] = 0.f;
  // forward bridges: groups by start ws = i * cf
  for (int i = 0; i < g.C; ++i) {
    const int start = i * g.cf;
    int tmax = -1;
    for (int t = 0; t < g.F; ++t) {
      int i_f, ws, i_r, we;
      readout_indices(g, t, i_f, ws, i_r, we);
      if (ws == start) tmax = t;
    }
    if (tmax < start) continue;
    float r = 0.f;
    for (int f = tmax; f >= start; --f) {
      int i_f, ws, i_r, we;
      readout_indices(g, f, i_f, ws, i_r, we);
      r = (f < tmax ? al[(size_t)(f + 1) * D] * r : 0.f) + (ws == start ? dDf[(size_t)f * D] : 0.f);
      R[(size_t)f * D] = r;
    }
    float pre = 1.f;
    for (int f = start; f <= tmax; ++f) {
      da[(size_t)f * D] += pre * R[(size_t)f * D];
      pre *= al[(size_t)f * D];
    }
  }
  // reverse bridges: groups by end we = min(i * cf, F) - 1
  for (int i = 1; i <= g.C; ++i) {
    const int end = min(i * g.cf, g.F) - 1;
    int tmin = g.F;
    for (int t = g.F - 1; t >= 0; --t) {
      int i_f, ws, i_r, we;
      readout_indices(g, t, i_f, ws, i_r, we);
      if (we == end) tmin = t;
    }
    if (tmin > end) continue;
    float r = 0.f;
    for (int f = tmin; f <= end; ++f) {
      int i_f, ws, i_r, we;
      readout_indices(g, f, i_f, ws, i_r, we);
      r = (f > tmin ? al[(size_t)(f - 1) * D] * r : 0.f) + (we == end ? dDr[(size_t)f * D] : 0.f);
      R[(size_t)f * D] = r;
    }
    float suf = 1.f;
    for (int f = end; f >= tmin; --f) {
      da[(size_t)f * D] += suf * R[(size_t)f * D];
      suf *= al[(size_t)f * D];
    }
  }
}

// ---------------------------------------------------------------------------
// Chain helpers for kernels 4-6: a D x D fp32 left factor staged in LDS
// (pitch D + 1), a 32-column block Y [D][32] in LDS.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ void stage_left(float* Ls, const float* src, bool transpose) {
  for (int e = threadIdx.x; e < D * D; e += 256) {
    const int r = e / D, c = e % D;
    if (transpose) Ls[c * (D + 1) + r] = src[e];
    else Ls[r * (D + 1) + c] = src[e];
  }
}

// Yout = Ls * Yin (+ add columns col0.. of a row-major D x D matrix).
template <int D>
__device__ __forceinline__ void left_mul(const float* Ls, const float* Yin, float* Yout,
                                         const float* add, int col0, int ncols) {
  constexpr int RPT = (D + 31) / 32;
  const int tx = threadIdx.x & 7, ty = threadIdx.x >> 3;
  float acc[RPT][4];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
  for (int kk = 0; kk < D; ++kk) {
    const f32x4 y = *reinterpret_cast<const f32x4*>(&Yin[kk * kBCB + tx * 4]);
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int row = ty + 32 * r;
      const float l = row < D ? Ls[row * (D + 1) + kk] : 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(l, y[c], acc[r][c]);
    }
  }
#pragma unroll
  for (int r = 0; r < RPT; ++r) {
    const int row = ty + 32 * r;
    if (row >= D) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int col = tx * 4 + c;
      float v = acc[r][c];
      if (add && col < ncols) v += add[(size_t)row * D + col0 + col];
      Yout[row * kBCB + col] = v;
    }
  }
}

template <int D>
__device__ __forceinline__ void load_block(float* Y, const float* src, int col0, int ncols, float scale) {
  for (int e = threadIdx.x; e < D * kBCB; e += 256) {
    const int r = e / kBCB, c = e % kBCB;
    Y[e] = c < ncols ? scale * src[(size_t)r * D + col0 + c] : 0.f;
  }
}

template <int D>
__device__ __forceinline__ void store_block(float* dst, const float* Y, int col0, int ncols) {
  for (int e = threadIdx.x; e < D * kBCB; e += 256) {
    const int r = e / kBCB, c = e % kBCB;
    if (c < ncols) dst[(size_t)r * D + col0 + c] = Y[e];
  }
}

// ---------------------------------------------------------------------------
// 4. Chunk-level adjoint scan, one workgroup per (b, h, direction, column
//    block).  Forward scan P[c+1] = T_c P[c] + U_c gives
//      mu[C] = dP[C],  mu[c] = dP[c] + T_c^T mu[c+1];
//    reverse scan P[c] = T_c P[c+1] + U_c gives
//      mu[0] = dP[0],  mu[c+1] = dP[c+1] + T_c^T mu[c].
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void vda_bwd_chunk_adjoint_kernel(VdaBwdArgs<T> a) {
  __shared__ __attribute__((aligned(16))) float smem[D * (D + 1) + 2 * D * kBCB];
  float* Ls = smem;
  float* Y0 = smem + D * (D + 1);
  float* Y1 = Y0 + D * kBCB;
  constexpr int NCB = (D + kBCB - 1) / kBCB;
  const Geometry& g = a.g;
  int id = blockIdx.x;
  const int cb = id % NCB; id /= NCB;
  const int dir = id % 2;
  const int bh = id / 2;
  const size_t DD = (size_t)D * D;
  const int col0 = cb * kBCB, ncols = min(kBCB, D - col0);
  const float* dP = a.dP + ((size_t)bh * 2 + dir) * (g.C + 1) * DD;
  float* mu = a.mu + ((size_t)bh * 2 + dir) * (g.C + 1) * DD;
  const int first = dir == 0 ? g.C : 0;
  load_block<D>(Y0, dP + (size_t)first * DD, col0, ncols, 1.f);
  __syncthreads();
  store_block<D>(mu + (size_t)first * DD, Y0, col0, ncols);
  float* yin = Y0;
  float* yout = Y1;
  for (int n = 0; n < g.C; ++n) {
    const int c = dir == 0 ? g.C - 1 - n : n;        // chunk whose map is applied
    const int slot = dir == 0 ? c : c + 1;           // adjoint produced
    __syncthreads();
    stage_left<D>(Ls, a.Tc + (((size_t)bh * 2 + dir) * g.C + c) * DD, true);
    __syncthreads();
    left_mul<D>(Ls, yin, yout, dP + (size_t)slot * DD, col0, ncols);
    __syncthreads();
    store_block<D>(mu + (size_t)slot * DD, yout, col0, ncols);
    float* tmp = yin; yin = yout; yout = tmp;
  }
}

// ---------------------------------------------------------------------------
// 5. Text state adjoint: dS_text = s (mu_fwd[0] + mu_rev[C]); Z_text = X_text dS_text.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void vda_bwd_text_kernel(VdaBwdArgs<T> a) {
  __shared__ __attribute__((aligned(16))) float smem[D * (D + 1) + 2 * D * kBCB];
  float* Ls = smem;
  float* Y0 = smem + D * (D + 1);
  float* Y1 = Y0 + D * kBCB;
  constexpr int NCB = (D + kBCB - 1) / kBCB;
  const Geometry& g = a.g;
  const int cb = blockIdx.x % NCB, bh = blockIdx.x / NCB;
  const size_t DD = (size_t)D * D;
  const int col0 = cb * kBCB, ncols = min(kBCB, D - col0);
  const float* m0 = a.mu + ((size_t)bh * 2 + 0) * (g.C + 1) * DD;
  const float* m1 = a.mu + (((size_t)bh * 2 + 1) * (g.C + 1) + g.C) * DD;
  for (int e = threadIdx.x; e < D * kBCB; e += 256) {
    const int r = e / kBCB, c = e % kBCB;
    Y0[e] = c < ncols ? a.init_scale * (m0[(size_t)r * D + col0 + c] + m1[(size_t)r * D + col0 + c]) : 0.f;
  }
  stage_left<D>(Ls, a.Xf + ((size_t)bh * (g.F + 1) + g.F) * DD, false);
  __syncthreads();
  left_mul<D>(Ls, Y0, Y1, nullptr, col0, ncols);
  __syncthreads();
  store_block<D>(a.ZT + (size_t)bh * DD, Y1, col0, ncols);
}

// ---------------------------------------------------------------------------
// 6. Frame states and frame adjoints of one chunk, one workgroup per
//    (b, h, direction, chunk, column block).
//    States: Sst[0][p] = forward state before frame p (p = 0..F), Sst[1][p]
//    = reverse state after frame p (p = 0..F, p = F the initial state).
//    The chunk writes its boundary copy and recomputes the states inside it.
//    Adjoints: Zst[dir][f] = X_f lambda_f (lambda_f for an anchor frame).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void vda_bwd_frame_adjoint_kernel(VdaBwdArgs<T> a,
                                                                    const float* __restrict__ Tf,
                                                                    const float* __restrict__ Uf) {
  __shared__ __attribute__((aligned(16))) float smem[D * (D + 1) + 2 * D * kBCB];
  float* Ls = smem;
  float* Y0 = smem + D * (D + 1);
  float* Y1 = Y0 + D * kBCB;
  constexpr int NCB = (D + kBCB - 1) / kBCB;
  const Geometry& g = a.g;
  int id = blockIdx.x;
  const int cb = id % NCB; id /= NCB;
  const int c = id % g.C; id /= g.C;
  const int dir = id % 2;
  const int bh = id / 2;
  const size_t DD = (size_t)D * D;
  const int col0 = cb * kBCB, ncols = min(kBCB, D - col0);
  const int f0 = c * g.cf, f1 = f0 + g.cf - 1;
  float* S = a.Sst + ((size_t)bh * 2 + dir) * (g.F + 1) * DD;
  float* Z = a.Zst + ((size_t)bh * 2 + dir) * g.F * DD;
  const float* P = (dir == 0 ? a.Pf : a.Pr) + (size_t)bh * (g.C + 1) * DD;
  const float* Tb = Tf + (size_t)bh * g.F * DD;
  const float* Ub = Uf + (size_t)bh * g.F * DD;
  const float* Xb = a.Xf + (size_t)bh * (g.F + 1) * DD;
  const float* al = a.alpha + (size_t)bh * g.F * D;

  // ---- states ----
  float* yin = Y0;
  float* yout = Y1;
  if (dir == 0) {
    load_block<D>(yin, P + (size_t)c * DD, col0, ncols, 1.f);          // before frame f0
    __syncthreads();
    store_block<D>(S + (size_t)f0 * DD, yin, col0, ncols);
    if (c == g.C - 1) {
      __syncthreads();
      load_block<D>(yout, P + (size_t)g.C * DD, col0, ncols, 1.f);
      __syncthreads();
      store_block<D>(S + (size_t)g.F * DD, yout, col0, ncols);
    }
    for (int f = f0; f < f1; ++f) {                                    // before frames f0+1 .. f1
      __syncthreads();
      stage_left<D>(Ls, Tb + (size_t)f * DD, false);
      __syncthreads();
      left_mul<D>(Ls, yin, yout, Ub + (size_t)f * DD, col0, ncols);
      __syncthreads();
      store_block<D>(S + (size_t)(f + 1) * DD, yout, col0, ncols);
      float* tmp = yin; yin = yout; yout = tmp;
    }
  } else {
    load_block<D>(yout, P + (size_t)c * DD, col0, ncols, 1.f);         // after frame f0
    __syncthreads();
    store_block<D>(S + (size_t)f0 * DD, yout, col0, ncols);
    load_block<D>(yin, P + (size_t)(c + 1) * DD, col0, ncols, 1.f);    // after frame f1 + 1
    __syncthreads();
    if (c == g.C - 1) store_block<D>(S + (size_t)g.F * DD, yin, col0, ncols);
    for (int f = f1; f > f0; --f) {                                    // after frames f1 .. f0+1
      __syncthreads();
      stage_left<D>(Ls, Tb + (size_t)f * DD, false);
      __syncthreads();
      left_mul<D>(Ls, yin, yout, Ub + (size_t)f * DD, col0, ncols);
      __syncthreads();
      store_block<D>(S + (size_t)f * DD, yout, col0, ncols);
      float* tmp = yin; yin = yout; yout = tmp;
    }
  }

  // ---- adjoints ----
  __syncthreads();
  const float* mu = a.mu + ((size_t)bh * 2 + dir) * (g.C + 1) * DD;
  yin = Y0;
  yout = Y1;
  load_block<D>(yin, mu + (size_t)(dir == 0 ? c + 1 : c) * DD, col0, ncols, 1.f);
  for (int n = 0; n < g.cf; ++n) {
    const int f = dir == 0 ? f1 - n : f0 + n;
    __syncthreads();                                   // yin = lambda_f
    if (!is_anchor_frame(g, f)) {
      stage_left<D>(Ls, Xb + (size_t)f * DD, false);
      __syncthreads();
      left_mul<D>(Ls, yin, yout, nullptr, col0, ncols);
      __syncthreads();
      float* tmp = yin; yin = yout; yout = tmp;        // yin = Z_f
    }
    store_block<D>(Z + (size_t)f * DD, yin, col0, ncols);
    // next lambda = diag(alpha_f) Z_f (each element read and rewritten by one thread)
    for (int e = threadIdx.x; e < D * kBCB; e += 256) yin[e] *= al[(size_t)f * D + e / kBCB];
  }
}

// ---------------------------------------------------------------------------
// 7. Per frame (and the text frame): dA_sym = -(Z0 S0^T + Z1 S1^T) + transpose,
//    dW = Z0 + Z1, the scan's alpha term, then the token gradients.  One
//    workgroup (256 threads) per (b, h, frame); dA_sym and dW sit in LDS
//    with pitch D + 1.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void vda_bwd_token_kernel(VdaBwdArgs<T> a) {
  constexpr int CPT = D / 16, TOK = 16, MP = D + 1, VC = 16, ZP = D + 4;
  __shared__ float Am[D * MP];
  __shared__ float Wm[D * MP];
  struct ZS { float z[VC][ZP]; float s[VC][ZP]; };
  struct KV { float k[TOK][MP]; float v[TOK][MP]; float b[TOK]; };
  __shared__ union { ZS zs; KV kv; } u;

  const Geometry& g = a.g;
  const int nfr = g.F + (g.T > 0 ? 1 : 0);
  const int f = blockIdx.x % nfr;
  const int bh = blockIdx.x / nfr;
  const int tid = threadIdx.x, grp = tid >> 4, sub = tid & 15;
  const int wave = tid >> 6, lane = tid & 63;
  const size_t DD = (size_t)D * D;
  const bool text = f == g.F;
  const float* Z0 = text ? a.ZT + (size_t)bh * DD : a.Zst + (((size_t)bh * 2 + 0) * g.F + f) * DD;
  const float* Z1 = text ? nullptr : a.Zst + (((size_t)bh * 2 + 1) * g.F + f) * DD;
  const float* S0 = text ? a.St + (size_t)bh * DD : a.Sst + (((size_t)bh * 2 + 0) * (g.F + 1) + f + 1) * DD;
  const float* S1 = text ? nullptr : a.Sst + (((size_t)bh * 2 + 1) * (g.F + 1) + f) * DD;

  // the scan's alpha term: rowsum(Z0 * S_fwd before f) + rowsum(Z1 * S_rev after f + 1)
  if (!text) {
    const float* P0 = a.Sst + (((size_t)bh * 2 + 0) * (g.F + 1) + f) * DD;
    const float* P1 = a.Sst + (((size_t)bh * 2 + 1) * (g.F + 1) + f + 1) * DD;
    for (int r = wave; r < D; r += 4) {
      float s = 0.f;
      for (int c = lane; c < D; c += 64)
        s += Z0[(size_t)r * D + c] * P0[(size_t)r * D + c] + Z1[(size_t)r * D + c] * P1[(size_t)r * D + c];
      s = sum64(s);
      if (lane == 0) a.dalpha[((size_t)bh * g.F + f) * D + r] += s;
    }
  }
  long long ntok;
  size_t tok0;
  const T *kp, *vp;
  const float* bp;
  T *dkp, *dvp;
  float* dbp;
  if (text) {
    ntok = g.T;
    tok0 = 0;
    kp = a.k_text + (size_t)bh * g.T * D;
    vp = a.v_text + (size_t)bh * g.T * D;
    bp = a.beta_text + (size_t)bh * g.T;
    dkp = a.dk_text + (size_t)bh * g.T * D;
    dvp = a.dv_text + (size_t)bh * g.T * D;
    dbp = a.dbeta_text + (size_t)bh * g.T;
  } else {
    ntok = g.N;
    tok0 = (size_t)bh * g.L + (size_t)f * g.N;
    kp = a.k + tok0 * D;
    vp = a.v + tok0 * D;
    bp = a.beta + tok0;
    dkp = a.dk + tok0 * D;
    dvp = a.dv + tok0 * D;
    dbp = a.dbeta + tok0;
  }
  if (!text && is_anchor_frame(g, f)) {            // no write: zero gradients
    for (long long e = tid; e < ntok * D; e += 256) {
      Elem<T>::store(dkp, e, 0.f);
      Elem<T>::store(dvp, e, 0.f);
    }
    for (long long n = tid; n < ntok; n += 256) dbp[n] = 0.f;
    return;
  }

  // dA = -(Z0 S0^T + Z1 S1^T): thread owns rows grp + 16 i, columns sub + 16 j
  float acc[CPT][CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i)
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc[i][j] = 0.f;
  for (int src = 0; src < (text ? 1 : 2); ++src) {
    const float* Zs = src ? Z1 : Z0;
    const float* Ss = src ? S1 : S0;
    for (int v0 = 0; v0 < D; v0 += VC) {
      __syncthreads();
      for (int e = tid; e < D * VC; e += 256) {
        const int r = e / VC, c = e % VC;
        u.zs.z[c][r] = Zs[(size_t)r * D + v0 + c];
        u.zs.s[c][r] = Ss[(size_t)r * D + v0 + c];
      }
      __syncthreads();
#pragma unroll 4
      for (int c = 0; c < VC; ++c) {
        float zi[CPT], sj[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) zi[i] = u.zs.z[c][grp + 16 * i];
#pragma unroll
        for (int j = 0; j < CPT; ++j) sj[j] = u.zs.s[c][sub + 16 * j];
#pragma unroll
        for (int i = 0; i < CPT; ++i)
#pragma unroll
          for (int j = 0; j < CPT; ++j) acc[i][j] = fmaf(zi[i], sj[j], acc[i][j]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < CPT; ++i)
#pragma unroll
    for (int j = 0; j < CPT; ++j) Am[(grp + 16 * i) * MP + sub + 16 * j] = -acc[i][j];
  for (int e = tid; e < D * D; e += 256) {
    const int r = e / D, c = e % D;
    Wm[r * MP + c] = Z0[e] + (Z1 ? Z1[e] : 0.f);
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < CPT; ++i)
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int r = grp + 16 * i, c = sub + 16 * j;
      acc[i][j] = Am[r * MP + c] + Am[c * MP + r];
    }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < CPT; ++i)
#pragma unroll
    for (int j = 0; j < CPT; ++j) Am[(grp + 16 * i) * MP + sub + 16 * j] = acc[i][j];

  // tokens: E = k dA_sym, Fm = k dW, Gm = v dW^T
  for (long long n0 = 0; n0 < ntok; n0 += TOK) {
    __syncthreads();
    for (int e = tid; e < TOK * D; e += 256) {
      const int r = e / D, c = e % D;
      const bool ok = n0 + r < ntok;
      u.kv.k[r][c] = ok ? Elem<T>::load(kp, (size_t)(n0 + r) * D + c) : 0.f;
      u.kv.v[r][c] = ok ? Elem<T>::load(vp, (size_t)(n0 + r) * D + c) : 0.f;
    }
    if (tid < TOK) u.kv.b[tid] = n0 + tid < ntok ? bp[n0 + tid] : 0.f;
    __syncthreads();
    float E[CPT], Fm[CPT], Gm[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) E[j] = Fm[j] = Gm[j] = 0.f;
    for (int kk = 0; kk < D; ++kk) {
      const float kv = u.kv.k[grp][kk], vv = u.kv.v[grp][kk];
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        E[j] = fmaf(kv, Am[kk * MP + sub + 16 * j], E[j]);
        Fm[j] = fmaf(kv, Wm[kk * MP + sub + 16 * j], Fm[j]);
        Gm[j] = fmaf(vv, Wm[(sub + 16 * j) * MP + kk], Gm[j]);
      }
    }
    const float b = u.kv.b[grp];
    float db = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = sub + 16 * j;
      db = fmaf(0.5f * E[j], u.kv.k[grp][c], db);
      db = fmaf(Fm[j], u.kv.v[grp][c], db);
    }
    db = sum16(db);
    const long long n = n0 + grp;
    if (n < ntok) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = sub + 16 * j;
        Elem<T>::store(dkp, (size_t)n * D + c, b * (E[j] + Gm[j]));
        Elem<T>::store(dvp, (size_t)n * D + c, b * Fm[j]);
      }
      if (sub == 0) dbp[n] = db;
    }
  }
}

// 8. dgamma = sum of the per-(b, h, frame) partial sums.
template <int D>
__global__ __launch_bounds__(128) void vda_bwd_dgamma_kernel(const float* __restrict__ dgp, long long rows,
                                                             float* __restrict__ dgamma) {
  const int c = threadIdx.x;
  if (c >= D) return;
  float s = 0.f;
  for (long long r = 0; r < rows; ++r) s += dgp[r * D + c];
  dgamma[c] = s;
}

template <typename T, int D>
hipError_t launch_all(const VdaBwdArgs<T>& a, const float* Tf, const float* Uf, float* dgamma,
                      hipStream_t s) {
  const Geometry& g = a.g;
  const unsigned BH = (unsigned)(g.B * g.H);
  constexpr int NCB = (D + kBCB - 1) / kBCB;
  vda_bwd_readout_kernel<T, D><<<BH * g.F, 256, 0, s>>>(a);
  vda_bwd_dp_kernel<T, D><<<BH * 2 * (g.C + 1), 256, 0, s>>>(a);
  vda_bwd_alpha_bridge_kernel<T, D><<<BH, 128, 0, s>>>(a);
  vda_bwd_chunk_adjoint_kernel<T, D><<<BH * 2 * NCB, 256, 0, s>>>(a);
  if (g.T > 0) vda_bwd_text_kernel<T, D><<<BH * NCB, 256, 0, s>>>(a);
  vda_bwd_frame_adjoint_kernel<T, D><<<BH * 2 * g.C * NCB, 256, 0, s>>>(a, Tf, Uf);
  vda_bwd_token_kernel<T, D><<<BH * (g.F + (g.T > 0 ? 1 : 0)), 256, 0, s>>>(a);
  if (dgamma && a.dgp) vda_bwd_dgamma_kernel<D><<<1, 128, 0, s>>>(a.dgp, (long long)BH * g.F, dgamma);
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_vda_bwd(const Geometry& g, const VdaBwdPtrs& p, const T* q, const T* k, const T* v,
                          const T* k_text, const T* v_text, const T* d_out, T* dq, T* dk, T* dv,
                          T* dk_text, T* dv_text, float eps, float init_scale, hipStream_t s) {
  VdaBwdArgs<T> a{g, q, k, v, p.beta, p.alpha, k_text, v_text, p.beta_text, p.g_l, p.gamma, d_out,
                  eps, init_scale, p.Pf, p.Pr, p.St, p.Xf, p.Tc, p.G, p.Dbr, p.dDbr,
                  p.dgamma ? p.dgp : nullptr, p.dP, p.mu, p.Sst, p.Zst, p.ZT, p.Rscr, dq, dk, dv,
                  p.dbeta, p.dalpha, dk_text, dv_text, p.dbeta_text, p.dg_l};
  switch (g.D) {
    case 16: return launch_all<T, 16>(a, p.Tf, p.Uf, p.dgamma, s);
    case 32: return launch_all<T, 32>(a, p.Tf, p.Uf, p.dgamma, s);
    case 64: return launch_all<T, 64>(a, p.Tf, p.Uf, p.dgamma, s);
    case 128: return launch_all<T, 128>(a, p.Tf, p.Uf, p.dgamma, s);
    default: return hipErrorInvalidValue;
  }
}

template hipError_t launch_vda_bwd<float>(const Geometry&, const VdaBwdPtrs&, const float*, const float*,
                                          const float*, const float*, const float*, const float*,
                                          float*, float*, float*, float*, float*, float, float,
                                          hipStream_t);
template hipError_t launch_vda_bwd<bf16_t>(const Geometry&, const VdaBwdPtrs&, const bf16_t*,
                                           const bf16_t*, const bf16_t*, const bf16_t*, const bf16_t*,
                                           const bf16_t*, bf16_t*, bf16_t*, bf16_t*, bf16_t*, bf16_t*,
                                           float, float, hipStream_t);

}  // namespace vdn
