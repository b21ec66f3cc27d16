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

#include <type_traits>

namespace vdn {

namespace {

constexpr int kBCB = 32;   // state columns per workgroup in the chain kernels
constexpr int kBridgeCh = 2;   // channels per workgroup of the bridge-alpha kernel (<= 56 F bytes of LDS)

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

// bf16 kernel (D = 64, 128) on v_mfma_f32_32x32x16_bf16.  NW waves; wave w
// owns the channel block vb = w % (D/32) of the 32-token sub-tile w / (D/32)
// of a 64-token step.  M = diag(D_f) P_f + diag(D_r) P_r is formed once per
// frame into LDS as bf16 hi + lo, row-major [k][v], so no wave holds
// fragments of it for the whole frame:
//   O^T  = M^T Q^T   (rows v of its block; M^T read from M with the
//                     transposing LDS read),
//   the RMSNorm / gate adjoint (three per-token sums exchanged through LDS),
//   dq^T = M dO^T    (rows k of block vb straight from M; dO rows from LDS),
//   G   += Q^T dO    (its G blocks, contracted over the step's tokens; both
//                     operands read transposed from the Q and dO row tiles).
// At the end G goes to memory and the bridge adjoints are row sums of
// G * P; dgamma partials are reduced through LDS.
template <int D> struct BwdReadoutShape {
  static constexpr int NW = D == 128 ? 8 : 4;   // waves per workgroup
};
template <int D>
__global__ __launch_bounds__(BwdReadoutShape<D>::NW * 64) void vda_bwd_readout_mfma_kernel(VdaBwdArgs<bf16_t> a) {
  constexpr int NB = D / 32, NKK = D / 16, NW = BwdReadoutShape<D>::NW, NT = NW * 64;
  constexpr int SUBT = NW / NB, TPS = 32 * SUBT;   // token sub-tiles and tokens per step
  // pitch (bf16) of the row tiles: 16-byte reads of 32 rows and transposing
  // reads of 4 rows x 64 bytes per half-wave are free of bank conflicts
  constexpr int DP = D == 128 ? 152 : 72;
  constexpr int NGB = NB * NB / NW;                // G blocks per wave
  static_assert(NGB * NW == NB * NB && TPS == 64, "work split");
  // G goes through LDS in NPASS slices of RPP rows at the end of the frame,
  // in the space the loop's tiles held
  constexpr int NPASS = D > 64 ? 2 : 1, RPP = D / NPASS;
  struct Loop {
    bf16_t mh[D * DP];        // M hi / lo, row-major [k][v]
    bf16_t ml[D * DP];
    bf16_t doh[TPS * DP];     // dO of the step, hi / lo
    bf16_t dol[TPS * DP];
  };
  struct Tail {
    float pd[RPP * (D + 1)];  // a slice of G
    float gsum[SUBT][D][33];  // dgamma partials
  };
  __shared__ __attribute__((aligned(16))) union {
    Loop t;
    Tail e;
  } u;
  __shared__ __attribute__((aligned(16))) bf16_t qrow[2][TPS * DP];   // the step's Q rows
  __shared__ float red[NW][32][3];
  __shared__ float dfs[D], drs[D];
  __shared__ __attribute__((aligned(16))) float gms[D];

  const Geometry& g = a.g;
  const int t = blockIdx.x % g.F;
  const int bh = blockIdx.x / g.F;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hg = lane >> 5, l32 = lane & 31;
  const int grp = lane >> 4, sl = lane & 15;       // 16-lane group of the transposing reads
  const int vb = wave % NB, ts = wave / NB;
  const size_t DD = (size_t)D * D;
  int i_f, ws, i_r, we;
  readout_indices(g, t, i_f, ws, i_r, we);
  const float* al = a.alpha + (size_t)bh * g.F * D;
  // bridges: thread (part, c) multiplies the decays of one direction's span
  // in frame order, with four frames' loads in flight together
  if (tid < 2 * D) {
    const int c = tid % D, part = tid / D;
    const int f0 = part == 0 ? ws : t, f1 = part == 0 ? t : we;   // inclusive
    float d = 1.f;
    int f = f0;
    for (; f + 3 <= f1; f += 4) {
      const float a0 = al[(size_t)f * D + c], a1 = al[(size_t)(f + 1) * D + c];
      const float a2 = al[(size_t)(f + 2) * D + c], a3 = al[(size_t)(f + 3) * D + c];
      d *= a0;
      d *= a1;
      d *= a2;
      d *= a3;
    }
    for (; f <= f1; ++f) d *= al[(size_t)f * D + c];
    (part == 0 ? dfs : drs)[c] = d;
    a.Dbr[(((size_t)bh * 2 + part) * g.F + t) * D + c] = d;
  }
  for (int c = tid; c < D; c += NT) gms[c] = a.gamma ? a.gamma[c] : 1.f;
  __syncthreads();
  const float* pf = a.Pf + ((size_t)bh * (g.C + 1) + i_f) * DD;
  const float* pr = a.Pr + ((size_t)bh * (g.C + 1) + i_r) * DD;
  // M[k][v] = D_f[k] P_f[k][v] + D_r[k] P_r[k][v] -> LDS as bf16 hi + lo,
  // four columns per thread and item
  for (int e = tid; e < D * D / 4; e += NT) {
    const int k = e / (D / 4), v0 = (e % (D / 4)) * 4;
    const f32x4 x4 = *reinterpret_cast<const f32x4*>(pf + (size_t)k * D + v0);
    const f32x4 y4 = *reinterpret_cast<const f32x4*>(pr + (size_t)k * D + v0);
    const float fk = dfs[k], rk = drs[k];
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2) {
      const float m0 = fk * x4[2 * p2] + rk * y4[2 * p2];
      const float m1 = fk * x4[2 * p2 + 1] + rk * y4[2 * p2 + 1];
      const float h0 = bf16_to_f32(f32_to_bf16(m0)), h1 = bf16_to_f32(f32_to_bf16(m1));
      hw[p2] = pack_bf16x2(h0, h1);
      lw[p2] = pack_bf16x2(m0 - h0, m1 - h1);
    }
    *reinterpret_cast<u32x2*>(&u.t.mh[k * DP + v0]) = u32x2{hw[0], hw[1]};
    *reinterpret_cast<u32x2*>(&u.t.ml[k * DP + v0]) = u32x2{lw[0], lw[1]};
  }
  const int bidx = bh / g.H, h = bh % g.H;
  const size_t tok0 = (size_t)bh * g.L + (size_t)t * g.N;
  f32x16 G[NGB];
#pragma unroll
  for (int b = 0; b < NGB; ++b) G[b] = f32x16{};
  float gacc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) gacc[i] = 0.f;

  // the next step's Q rows travel global -> registers -> LDS (qrow) while
  // the current step runs: CQ 16-byte chunks per thread
  constexpr int CQ = TPS * D / 8 / NT;
  u32x4 qst[CQ];
  auto fetch_q = [&](int n0) {
#pragma unroll
    for (int i = 0; i < CQ; ++i) {
      const int c = threadIdx.x + NT * i;
      const int r = c / (D / 8), c8 = c % (D / 8);
      qst[i] = n0 + r < g.N ? ld16(a.q + (tok0 + n0 + r) * D + c8 * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto stage_q = [&](int b) {
#pragma unroll
    for (int i = 0; i < CQ; ++i) {
      const int c = threadIdx.x + NT * i;
      st16(&qrow[b][(c / (D / 8)) * DP + (c % (D / 8)) * 8], qst[i]);
    }
  };
  const int nl = ts * 32 + l32;                 // token within the step
  // dOhat of this lane's token and 16 channels, the next step's requested early
  u32x2 dx[4], dxn[4];
  auto load_do = [&](int n, u32x2* dst) {
    const bf16_t* dob = a.d_out + (((size_t)bidx * g.L + (size_t)t * g.N + n) * g.H + h) * D + vb * 32;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4)
      dst[i4] = n < g.N ? *reinterpret_cast<const u32x2*>(dob + 8 * i4 + 4 * hg) : u32x2{0, 0};
  };
  // the gate of this lane's token, also requested a step early: a load
  // issued and consumed within one step would make the step wait for every
  // prefetch issued before it
  auto load_gate = [&](int n) { return n < g.N ? a.g_l[(size_t)bh * g.L + (size_t)t * g.N + n] : 0.f; };
  float gate_c = load_gate(nl), gate_n = 0.f;
  load_do(nl, dx);
  fetch_q(0);
  stage_q(0);
  __syncthreads();
  // transposing reads of M^T rows v of block vb: group lane sl points at row
  // k = 16 kk + 8 (grp / 2) + sl / 4 (+ 4), columns v = 32 vb + 16 (grp % 2) + 4 (sl % 4)
  const int mt_off = (8 * (grp >> 1) + (sl >> 2)) * DP + vb * 32 + 16 * (grp & 1) + 4 * (sl & 3);
  // G operands: rows 16 (grp % 2) + 0..15 of a block, contraction slots
  // 8 (grp / 2) + 0..7, four tokens a read
  const int trow = 8 * (grp >> 1) + (sl >> 2), tcol = 16 * (grp & 1) + 4 * (sl & 3);
  for (int n0 = 0, st = 0; n0 < g.N; n0 += TPS, st ^= 1) {
    const int n = n0 + nl;
    const bool valid = n < g.N;
    const bool more = n0 + TPS < g.N;
    if (more) fetch_q(n0 + TPS);
    load_do(n + TPS, dxn);
    gate_n = load_gate(n + TPS);
    // O^T block
    f32x16 o = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const bf16x8 qf = as_bf16x8(ld16(&qrow[st][nl * DP + kk * 16 + hg * 8]));
      const bf16_t* ph = &u.t.mh[kk * 16 * DP + mt_off];
      const bf16_t* pl = &u.t.ml[kk * 16 * DP + mt_off];
      const u32x2 h0 = lds_read_tr16(ph), h1 = lds_read_tr16(ph + 4 * DP);
      const u32x2 l0 = lds_read_tr16(pl), l1 = lds_read_tr16(pl + 4 * DP);
      o = mfma32x32x16(as_bf16x8(u32x4{h0[0], h0[1], h1[0], h1[1]}), qf, o);
      o = mfma32x32x16(as_bf16x8(u32x4{l0[0], l0[1], l1[0], l1[1]}), qf, o);
    }
    // the token's three sums over its channels, from O directly (1 / r
    // factors out of the last two), exchanged once: |o|^2, sum dOhat gamma o,
    // sum u o with u = g_l gamma dOhat
    const float gate = gate_c;
    const f32x4* gq = reinterpret_cast<const f32x4*>(&gms[vb * 32 + 4 * hg]);
    float u_[16], ss = 0.f, dgr = 0.f, uor = 0.f;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const u32x2 x = dx[i4];
      const float dv4[4] = {bf16_to_f32((bf16_t)(x[0] & 0xFFFFu)), bf16_to_f32((bf16_t)(x[0] >> 16)),
                            bf16_to_f32((bf16_t)(x[1] & 0xFFFFu)), bf16_to_f32((bf16_t)(x[1] >> 16))};
      const f32x4 gm4 = gq[2 * i4];                    // gamma of channels 8 i4 + 4 hg + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * i4 + r;
        ss = fmaf(o[i], o[i], ss);
        u_[i] = gate * gm4[r] * dv4[r];
        dgr = fmaf(dv4[r] * gm4[r], o[i], dgr);
        uor = fmaf(u_[i], o[i], uor);
      }
    }
    ss = half_sum(ss);
    dgr = half_sum(dgr);
    uor = half_sum(uor);
    if (hg == 0) {
      red[wave][l32][0] = ss;
      red[wave][l32][1] = dgr;
      red[wave][l32][2] = uor;
    }
    lds_barrier();
    float sst = 0.f, dgt = 0.f, uyt = 0.f;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      sst += red[ts * NB + b][l32][0];
      dgt += red[ts * NB + b][l32][1];
      uyt += red[ts * NB + b][l32][2];
    }
    const float inv = rsqrtf(sst / (float)D + a.eps);
    dgt *= inv;
    uyt *= inv;
    const size_t l = (size_t)t * g.N + n;
    if (vb == 0 && hg == 0 && valid && a.dg_l) a.dg_l[(size_t)bh * g.L + l] = dgt;
    const float muy = uyt / (float)D;
    // y = o / r, the dgamma partials, dO of this block -> LDS as hi + lo
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const u32x2 x = dx[i4];
      const float dv4[4] = {bf16_to_f32((bf16_t)(x[0] & 0xFFFFu)), bf16_to_f32((bf16_t)(x[0] >> 16)),
                            bf16_to_f32((bf16_t)(x[1] & 0xFFFFu)), bf16_to_f32((bf16_t)(x[1] >> 16))};
      uint32_t ph[2], pl[2];
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2) {
        float hv[2], lv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int i = 4 * i4 + 2 * r2 + e;
          const float y = valid ? o[i] * inv : 0.f;
          gacc[i] = fmaf(dv4[2 * r2 + e] * gate, y, gacc[i]);
          const float d = valid ? inv * (u_[i] - y * muy) : 0.f;
          hv[e] = bf16_to_f32(f32_to_bf16(d));
          lv[e] = d - hv[e];
        }
        ph[r2] = pack_bf16x2(hv[0], hv[1]);
        pl[r2] = pack_bf16x2(lv[0], lv[1]);
      }
      const int c0 = vb * 32 + 8 * i4 + 4 * hg;
      *reinterpret_cast<u32x2*>(&u.t.doh[nl * DP + c0]) = u32x2{ph[0], ph[1]};
      *reinterpret_cast<u32x2*>(&u.t.dol[nl * DP + c0]) = u32x2{pl[0], pl[1]};
    }
    // the next step's Q rows go to the other buffer (last read in the
    // previous step, before this step's first barrier); the barrier below
    // publishes them with dO
    if (more) stage_q(st ^ 1);
    lds_barrier();
    // dq^T rows k of block vb for the sub-tile's tokens
    f32x16 dq = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int mo = (vb * 32 + l32) * DP + kk * 16 + hg * 8;
      const bf16x8 mh_ = as_bf16x8(ld16(&u.t.mh[mo]));
      const bf16x8 ml_ = as_bf16x8(ld16(&u.t.ml[mo]));
      const bf16x8 bh_ = as_bf16x8(ld16(&u.t.doh[nl * DP + kk * 16 + hg * 8]));
      const bf16x8 bl_ = as_bf16x8(ld16(&u.t.dol[nl * DP + kk * 16 + hg * 8]));
      dq = mfma32x32x16(mh_, bh_, dq);
      dq = mfma32x32x16(ml_, bh_, dq);
      dq = mfma32x32x16(mh_, bl_, dq);
    }
    if (valid) {
      bf16_t* dqr = a.dq + (tok0 + n) * D + vb * 32;
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        u32x2 pk;
        pk[0] = pack_bf16x2(dq[4 * i4 + 0], dq[4 * i4 + 1]);
        pk[1] = pack_bf16x2(dq[4 * i4 + 2], dq[4 * i4 + 3]);
        *reinterpret_cast<u32x2*>(dqr + 8 * i4 + 4 * hg) = pk;
      }
    }
    // G += Q^T dO over the step's tokens
#pragma unroll
    for (int b = 0; b < NGB; ++b) {
      const int blk = wave + NW * b;
      const int kb = blk / NB, vbg = blk % NB;
#pragma unroll
      for (int ns = 0; ns < TPS / 16; ++ns) {
        const int r0 = (ns * 16 + trow) * DP, r1 = r0 + 4 * DP;
        const bf16_t* qa = &qrow[st][kb * 32 + tcol];
        const bf16_t* dh = &u.t.doh[vbg * 32 + tcol];
        const bf16_t* dl = &u.t.dol[vbg * 32 + tcol];
        const u32x2 q0 = lds_read_tr16(qa + r0), q1 = lds_read_tr16(qa + r1);
        const u32x2 h0 = lds_read_tr16(dh + r0), h1 = lds_read_tr16(dh + r1);
        const u32x2 l0 = lds_read_tr16(dl + r0), l1 = lds_read_tr16(dl + r1);
        const bf16x8 aq = as_bf16x8(u32x4{q0[0], q0[1], q1[0], q1[1]});
        const bf16x8 bh_ = as_bf16x8(u32x4{h0[0], h0[1], h1[0], h1[1]});
        const bf16x8 bl_ = as_bf16x8(u32x4{l0[0], l0[1], l1[0], l1[1]});
        G[b] = mfma32x32x16(aq, bh_, G[b]);
        G[b] = mfma32x32x16(aq, bl_, G[b]);
      }
    }
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) dx[i4] = dxn[i4];
    gate_c = gate_n;
    // no barrier here: the next writes to the dO tiles and the sums follow
    // the next step's first barrier, which every wave reaches only after
    // this step's reads
  }
  __syncthreads();      // the tiles are read out before the tail reuses their space
  // G -> memory and, a slice of rows at a time, LDS; bridge adjoints
  // dD = rowsum(G * P)
  float* Go = a.G + ((size_t)bh * g.F + t) * DD;
#pragma unroll
  for (int i = 0; i < 16; ++i) u.e.gsum[ts][vb * 32 + mfma32_row(i, hg)][l32] = gacc[i];
#pragma unroll
  for (int ps = 0; ps < NPASS; ++ps) {
#pragma unroll
    for (int b = 0; b < NGB; ++b) {
      const int blk = wave + NW * b;
      const int kb = blk / NB, vbg = blk % NB;
      if (kb * 32 / RPP != ps) continue;      // wave-uniform
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int k = kb * 32 + mfma32_row(i, hg), v = vbg * 32 + l32;
        Go[(size_t)k * D + v] = G[b][i];
        u.e.pd[(k - ps * RPP) * (D + 1) + v] = G[b][i];
      }
    }
    __syncthreads();
    for (int rr = wave; rr < RPP; rr += NW) {
      const int r = ps * RPP + rr;
      float sf = 0.f, sr = 0.f;
      for (int c = lane; c < D; c += 64) {
        const float x = u.e.pd[rr * (D + 1) + c];
        sf = fmaf(x, pf[(size_t)r * D + c], sf);
        sr = fmaf(x, pr[(size_t)r * D + c], sr);
      }
      sf = sum64(sf);
      sr = sum64(sr);
      if (lane == 0) {
        a.dDbr[(((size_t)bh * 2 + 0) * g.F + t) * D + r] = sf;
        a.dDbr[(((size_t)bh * 2 + 1) * g.F + t) * D + r] = sr;
      }
    }
    if (ps + 1 < NPASS) __syncthreads();      // the slice is read before the next one lands
  }
  if (a.dgp) {
    for (int c = tid; c < D; c += NT) {
      float sg = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < SUBT; ++s2)
        for (int j = 0; j < 32; ++j) sg += u.e.gsum[s2][c][j];
      a.dgp[((size_t)bh * g.F + t) * D + c] = sg;
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
//    the reverse bridges t..we mirror this.  A workgroup takes 2 channels of
//    one (b, h): alpha, dD, R and the dalpha sums for all frames sit in LDS
//    (5 F floats per channel), one thread per channel runs the recurrences.
//    Writes (initialises) dalpha.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void vda_bwd_alpha_bridge_kernel(VdaBwdArgs<T> a) {
  // LDS: alpha, dD_fwd, dD_rev, R, sums (kBridgeCh floats per frame each),
  // then ws and we per frame and the groups' last / first query (ints)
  extern __shared__ float bsm[];
  const Geometry& g = a.g;
  constexpr int NG = D / kBridgeCh;
  const int grp = blockIdx.x % NG, bh = blockIdx.x / NG;
  const int c0 = grp * kBridgeCh;
  const int F = g.F, C = g.C;
  float* al = bsm;
  float* dDf = al + F * kBridgeCh;
  float* dDr = dDf + F * kBridgeCh;
  float* R = dDr + F * kBridgeCh;
  float* das = R + F * kBridgeCh;
  int* wsA = reinterpret_cast<int*>(das + F * kBridgeCh);
  int* weA = wsA + F;
  int* tmaxA = weA + F;            // [C]: last query with ws = i * cf
  int* tminA = tmaxA + C;          // [C + 1]: first query with we = min(i * cf, F) - 1
  const float* alg = a.alpha + (size_t)bh * F * D + c0;
  const float* dDfg = a.dDbr + ((size_t)bh * 2 + 0) * F * D + c0;
  const float* dDrg = a.dDbr + ((size_t)bh * 2 + 1) * F * D + c0;
  for (int e = threadIdx.x; e < F * kBridgeCh; e += 64) {
    const int f = e / kBridgeCh, c = e % kBridgeCh;
    al[e] = alg[(size_t)f * D + c];
    dDf[e] = dDfg[(size_t)f * D + c];
    dDr[e] = dDrg[(size_t)f * D + c];
    das[e] = 0.f;
  }
  for (int t = threadIdx.x; t < F; t += 64) {
    int i_f, ws, i_r, we;
    readout_indices(g, t, i_f, ws, i_r, we);
    wsA[t] = ws;
    weA[t] = we;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 0; i < C; ++i) tmaxA[i] = -1;
    for (int i = 0; i <= C; ++i) tminA[i] = F;
    for (int t = 0; t < F; ++t) tmaxA[wsA[t] / g.cf] = t;                   // ascending: the last wins
    for (int t = F - 1; t >= 0; --t) tminA[(weA[t] + 1 + g.cf - 1) / g.cf] = t;
  }
  __syncthreads();
  const int c = threadIdx.x;
  if (c >= kBridgeCh) return;
  auto A = [&](int f) { return al[f * kBridgeCh + c]; };
  // forward bridges: groups by start ws = i * cf
  for (int i = 0; i < C; ++i) {
    const int start = i * g.cf, tmax = tmaxA[i];
    if (tmax < start) continue;
    float r = 0.f;
    for (int f = tmax; f >= start; --f) {
      r = (f < tmax ? A(f + 1) * r : 0.f) + (wsA[f] == start ? dDf[f * kBridgeCh + c] : 0.f);
      R[f * kBridgeCh + c] = r;
    }
    float pre = 1.f;
    for (int f = start; f <= tmax; ++f) {
      das[f * kBridgeCh + c] += pre * R[f * kBridgeCh + c];
      pre *= A(f);
    }
  }
  // reverse bridges: groups by end we = min(i * cf, F) - 1
  for (int i = 1; i <= C; ++i) {
    const int end = min(i * g.cf, F) - 1, tmin = tminA[i];
    if (tmin > end) continue;
    float r = 0.f;
    for (int f = tmin; f <= end; ++f) {
      r = (f > tmin ? A(f - 1) * r : 0.f) + (weA[f] == end ? dDr[f * kBridgeCh + c] : 0.f);
      R[f * kBridgeCh + c] = r;
    }
    float suf = 1.f;
    for (int f = end; f >= tmin; --f) {
      das[f * kBridgeCh + c] += suf * R[f * kBridgeCh + c];
      suf *= A(f);
    }
  }
  float* da = a.dalpha + (size_t)bh * F * D + c0 + c;
  for (int f = 0; f < F; ++f) da[(size_t)f * D] = das[f * kBridgeCh + c];
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
// fp32 MFMA chains for kernels 4 and 6 (D = 64, 128), on
// v_mfma_f32_32x32x2f32.  A workgroup owns a 32-column block Y of the
// state (or adjoint), kept transposed in LDS (Yt[n][k]); wave w < D/32 owns
// rows 32w..32w+31 of each left factor, loaded from global memory straight
// into registers -- the next step's while the current product runs.  Lane
// half g takes k = 8j + 4g .. 8j + 4g + 3 of each 8-wide group on both
// operands.
// ---------------------------------------------------------------------------
template <int D>
struct ChainMfma {
  static constexpr int NB = D / 32, YP = D + 4, NK8 = D / 8;
  float* Yt;
  int col0, wave, hg, l32;
  bool mw;

  __device__ __forceinline__ ChainMfma(float* yt, int c0) : Yt(yt), col0(c0) {
    const int tid = threadIdx.x;
    wave = tid >> 6;
    hg = (tid & 63) >> 5;
    l32 = tid & 31;
    mw = wave < NB;
  }
  // rows of L (row-major) or of L^T (transposed: columns of L)
  __device__ __forceinline__ void load_left(const float* Lm, bool transposed, f32x4 (&dst)[NK8]) const {
    const int mrow = wave * 32 + l32;
#pragma unroll
    for (int j = 0; j < NK8; ++j) {
      if (!mw) { dst[j] = f32x4{}; continue; }
      const int k0 = 8 * j + 4 * hg;
      if (transposed)
        dst[j] = f32x4{Lm[(size_t)k0 * D + mrow], Lm[(size_t)(k0 + 1) * D + mrow],
                       Lm[(size_t)(k0 + 2) * D + mrow], Lm[(size_t)(k0 + 3) * D + mrow]};
      else
        dst[j] = *reinterpret_cast<const f32x4*>(Lm + (size_t)mrow * D + k0);
    }
  }
  __device__ __forceinline__ void y_from(const float* src, float scale = 1.f) const {
    for (int e = threadIdx.x; e < D * 32; e += 256) {
      const int k = e / 32, n = e % 32;
      Yt[n * YP + k] = scale * src[(size_t)k * D + col0 + n];
    }
  }
  __device__ __forceinline__ f32x16 product(const f32x4 (&lf)[NK8]) const {
    f32x16 acc = f32x16{};
#pragma unroll
    for (int j = 0; j < NK8; ++j) {
      const f32x4 yb = *reinterpret_cast<const f32x4*>(&Yt[l32 * YP + 8 * j + 4 * hg]);
#pragma unroll
      for (int q = 0; q < 4; ++q) acc = mfma32x32x2f32(lf[j][q], yb[q], acc);
    }
    return acc;
  }
  __device__ __forceinline__ f32x16 y_rows() const {     // the wave's rows of Y, accumulator layout
    f32x16 acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = Yt[l32 * YP + wave * 32 + mfma32_row(i, hg)];
    return acc;
  }
  __device__ __forceinline__ int row(int i) const { return wave * 32 + mfma32_row(i, hg); }
  __device__ __forceinline__ void to_y(const f32x16& acc) const {
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const f32x4 v = {acc[4 * i4], acc[4 * i4 + 1], acc[4 * i4 + 2], acc[4 * i4 + 3]};
      *reinterpret_cast<f32x4*>(&Yt[l32 * YP + wave * 32 + 8 * i4 + 4 * hg]) = v;
    }
  }
  __device__ __forceinline__ void to_global(const f32x16& acc, float* dst) const {
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[(size_t)row(i) * D + col0 + l32] = acc[i];
  }
};

// Kernel 4 on MFMA: grid (b, h, direction, column block).
template <typename T, int D>
__global__ __launch_bounds__(256) void vda_bwd_chunk_adjoint_mfma_kernel(VdaBwdArgs<T> a) {
  using CM = ChainMfma<D>;
  __shared__ __attribute__((aligned(16))) float Yt[32 * CM::YP];
  constexpr int NCB = D / 32;
  const Geometry& g = a.g;
  int id = blockIdx.x;
  const int cb = id % NCB; id /= NCB;
  const int dir = id % 2;
  const int bh = id / 2;
  const size_t DD = (size_t)D * D;
  CM cm(Yt, cb * 32);
  const float* dP = a.dP + ((size_t)bh * 2 + dir) * (g.C + 1) * DD;
  float* mu = a.mu + ((size_t)bh * 2 + dir) * (g.C + 1) * DD;
  const float* Tc = a.Tc + ((size_t)bh * 2 + dir) * g.C * DD;
  const int first = dir == 0 ? g.C : 0;
  cm.y_from(dP + (size_t)first * DD);
  for (int e = threadIdx.x; e < D * 32; e += 256) {
    const int k = e / 32, n = e % 32;
    mu[(size_t)first * DD + (size_t)k * D + cm.col0 + n] = dP[(size_t)first * DD + (size_t)k * D + cm.col0 + n];
  }
  f32x4 lf[CM::NK8], ln[CM::NK8];
  auto chunk = [&](int n) { return dir == 0 ? g.C - 1 - n : n; };
  cm.load_left(Tc + (size_t)chunk(0) * DD, true, lf);
  for (int n = 0; n < g.C; ++n) {
    const int c = chunk(n);
    const int slot = dir == 0 ? c : c + 1;
    if (n + 1 < g.C) cm.load_left(Tc + (size_t)chunk(n + 1) * DD, true, ln);
    __syncthreads();
    f32x16 acc = f32x16{};
    if (cm.mw) {
      acc = cm.product(lf);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += dP[(size_t)slot * DD + (size_t)cm.row(i) * D + cm.col0 + cm.l32];
    }
    __syncthreads();
    if (cm.mw) {
      cm.to_y(acc);
      cm.to_global(acc, mu + (size_t)slot * DD);
    }
#pragma unroll
    for (int j = 0; j < CM::NK8; ++j) lf[j] = ln[j];
  }
}

// Kernel 6 on MFMA: grid (b, h, direction, chunk, column block).
template <typename T, int D>
__global__ __launch_bounds__(256) void vda_bwd_frame_adjoint_mfma_kernel(VdaBwdArgs<T> a,
                                                                         const float* __restrict__ Tf,
                                                                         const float* __restrict__ Uf) {
  using CM = ChainMfma<D>;
  __shared__ __attribute__((aligned(16))) float Yt[32 * CM::YP];
  constexpr int NCB = D / 32;
  const Geometry& g = a.g;
  int id = blockIdx.x;
  const int cb = id % NCB; id /= NCB;
  const int c = id % g.C; id /= g.C;
  const int dir = id % 2;
  const int bh = id / 2;
  const size_t DD = (size_t)D * D;
  CM cm(Yt, cb * 32);
  const int f0 = c * g.cf, f1 = f0 + g.cf - 1;
  float* S = a.Sst + ((size_t)bh * 2 + dir) * (g.F + 1) * DD;
  float* Z = a.Zst + ((size_t)bh * 2 + dir) * g.F * DD;
  const float* P = (dir == 0 ? a.Pf : a.Pr) + (size_t)bh * (g.C + 1) * DD;
  const float* Tb = Tf + (size_t)bh * g.F * DD;
  const float* Ub = Uf + (size_t)bh * g.F * DD;
  const float* Xb = a.Xf + (size_t)bh * (g.F + 1) * DD;
  const float* al = a.alpha + (size_t)bh * g.F * D;

  // boundary copies: S[f0] = P[c]; the last chunk also writes S[F] = P[C]
  for (int e = threadIdx.x; e < D * 32; e += 256) {
    const size_t o = (size_t)(e / 32) * D + cm.col0 + e % 32;
    S[(size_t)f0 * DD + o] = P[(size_t)c * DD + o];
    if (c == g.C - 1) S[(size_t)g.F * DD + o] = P[(size_t)g.C * DD + o];
  }
  // ---- states inside the chunk ----
  const int nst = g.cf - 1;
  auto sframe = [&](int s2) { return dir == 0 ? f0 + s2 : f1 - s2; };
  f32x4 lf[CM::NK8], ln[CM::NK8];
  cm.y_from(P + (size_t)(dir == 0 ? c : c + 1) * DD);
  if (nst > 0) cm.load_left(Tb + (size_t)sframe(0) * DD, false, lf);
  for (int s2 = 0; s2 < nst; ++s2) {
    const int f = sframe(s2);
    if (s2 + 1 < nst) cm.load_left(Tb + (size_t)sframe(s2 + 1) * DD, false, ln);
    __syncthreads();
    f32x16 acc = f32x16{};
    if (cm.mw) {
      acc = cm.product(lf);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] += Ub[(size_t)f * DD + (size_t)cm.row(i) * D + cm.col0 + cm.l32];
    }
    __syncthreads();
    if (cm.mw) {
      cm.to_y(acc);
      cm.to_global(acc, S + (size_t)(dir == 0 ? f + 1 : f) * DD);
    }
#pragma unroll
    for (int j = 0; j < CM::NK8; ++j) lf[j] = ln[j];
  }
  // ---- adjoints: Z_f = X_f lambda_f (lambda_f for anchors), lambda <- diag(alpha_f) Z_f ----
  const float* mu = a.mu + ((size_t)bh * 2 + dir) * (g.C + 1) * DD;
  auto aframe = [&](int n) { return dir == 0 ? f1 - n : f0 + n; };
  __syncthreads();
  cm.y_from(mu + (size_t)(dir == 0 ? c + 1 : c) * DD);
  if (!is_anchor_frame(g, aframe(0))) cm.load_left(Xb + (size_t)aframe(0) * DD, false, lf);
  for (int n = 0; n < g.cf; ++n) {
    const int f = aframe(n);
    if (n + 1 < g.cf && !is_anchor_frame(g, aframe(n + 1)))
      cm.load_left(Xb + (size_t)aframe(n + 1) * DD, false, ln);
    __syncthreads();
    f32x16 acc = f32x16{};
    if (cm.mw) acc = is_anchor_frame(g, f) ? cm.y_rows() : cm.product(lf);
    __syncthreads();
    if (cm.mw) {
      cm.to_global(acc, Z + (size_t)f * DD);
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] *= al[(size_t)f * D + cm.row(i)];
      cm.to_y(acc);
    }
#pragma unroll
    for (int j = 0; j < CM::NK8; ++j) lf[j] = ln[j];
  }
}

// ---------------------------------------------------------------------------
// 7. Per frame (and the text frame): dA_sym = -(Z0 S0^T + Z1 S1^T) + transpose,
//    dW = Z0 + Z1, the scan's alpha term, then the token gradients.  One
//    workgroup (256 threads) per (b, h, frame).
// ---------------------------------------------------------------------------
template <typename T>
struct FrameTok {
  bool text, anchor;
  const float *Z0, *Z1, *S0, *S1;      // Z1 = S1 = nullptr for the text frame
  long long ntok;
  const T *kp, *vp;
  const float* bp;
  T *dkp, *dvp;
  float* dbp;
};

template <typename T, int D>
__device__ __forceinline__ FrameTok<T> frame_tok(const VdaBwdArgs<T>& a, int bh, int f) {
  const Geometry& g = a.g;
  const size_t DD = (size_t)D * D;
  FrameTok<T> r;
  r.text = f == g.F;
  r.anchor = !r.text && is_anchor_frame(g, f);
  if (r.text) {
    r.Z0 = a.ZT + (size_t)bh * DD;
    r.S0 = a.St + (size_t)bh * DD;
    r.Z1 = r.S1 = nullptr;
    r.ntok = g.T;
    r.kp = a.k_text + (size_t)bh * g.T * D;
    r.vp = a.v_text + (size_t)bh * g.T * D;
    r.bp = a.beta_text + (size_t)bh * g.T;
    r.dkp = a.dk_text + (size_t)bh * g.T * D;
    r.dvp = a.dv_text + (size_t)bh * g.T * D;
    r.dbp = a.dbeta_text + (size_t)bh * g.T;
  } else {
    r.Z0 = a.Zst + (((size_t)bh * 2 + 0) * g.F + f) * DD;
    r.Z1 = a.Zst + (((size_t)bh * 2 + 1) * g.F + f) * DD;
    r.S0 = a.Sst + (((size_t)bh * 2 + 0) * (g.F + 1) + f + 1) * DD;   // forward state after f
    r.S1 = a.Sst + (((size_t)bh * 2 + 1) * (g.F + 1) + f) * DD;       // reverse state after f
    r.ntok = g.N;
    const size_t tok0 = (size_t)bh * g.L + (size_t)f * g.N;
    r.kp = a.k + tok0 * D;
    r.vp = a.v + tok0 * D;
    r.bp = a.beta + tok0;
    r.dkp = a.dk + tok0 * D;
    r.dvp = a.dv + tok0 * D;
    r.dbp = a.dbeta + tok0;
  }
  return r;
}

// The scan's alpha term of a video frame, added to dalpha (initialised by
// the bridge kernel): rowsum(Z0 * forward state before f) + rowsum(Z1 *
// reverse state after f + 1).  256 / D threads per row, each a contiguous
// slice of columns; all loads are independent.
template <typename T, int D>
__device__ __forceinline__ void alpha_scan_term(const VdaBwdArgs<T>& a, const FrameTok<T>& ft, int bh,
                                                int f) {
  constexpr int TPR = 256 / D, CW = D / TPR;
  const Geometry& g = a.g;
  const size_t DD = (size_t)D * D;
  const int r = threadIdx.x / TPR, part = threadIdx.x % TPR;
  const size_t o = (size_t)r * D + part * CW;
  const float* z0 = ft.Z0 + o;
  const float* z1 = ft.Z1 + o;
  const float* p0 = a.Sst + (((size_t)bh * 2 + 0) * (g.F + 1) + f) * DD + o;
  const float* p1 = a.Sst + (((size_t)bh * 2 + 1) * (g.F + 1) + f + 1) * DD + o;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CW; ++c) s = fmaf(z0[c], p0[c], fmaf(z1[c], p1[c], s));
#pragma unroll
  for (int m = TPR / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m, TPR);
  if (part == 0) a.dalpha[((size_t)bh * g.F + f) * D + r] += s;
}

template <typename T>
__device__ __forceinline__ void zero_tokens(const FrameTok<T>& ft, int D) {
  for (long long e = threadIdx.x; e < ft.ntok * D; e += 256) {
    Elem<T>::store(ft.dkp, e, 0.f);
    Elem<T>::store(ft.dvp, e, 0.f);
  }
  for (long long n = threadIdx.x; n < ft.ntok; n += 256) ft.dbp[n] = 0.f;
}

// Staging of Z and S column slices for the dA product.
template <int D>
struct ZSStage {
  static constexpr int VC = 16, ZP = D + 4;
  float z[VC][ZP];
  float s[VC][ZP];
};

// acc[i][j] = (Z0 S0^T + Z1 S1^T)[grp + 16 i][sub + 16 j] (fp32, 256 threads).
template <int D>
__device__ __forceinline__ void frame_zst(const float* Z0, const float* S0, const float* Z1, const float* S1,
                                          ZSStage<D>& st, float (&acc)[D / 16][D / 16]) {
  constexpr int CPT = D / 16, VC = ZSStage<D>::VC;
  const int tid = threadIdx.x, grp = tid >> 4, sub = tid & 15;
#pragma unroll
  for (int i = 0; i < CPT; ++i)
#pragma unroll
    for (int j = 0; j < CPT; ++j) acc[i][j] = 0.f;
  for (int src = 0; src < (Z1 ? 2 : 1); ++src) {
    const float* Zs = src ? Z1 : Z0;
    const float* Ss = src ? S1 : S0;
    for (int v0 = 0; v0 < D; v0 += VC) {
      __syncthreads();
      for (int e = tid; e < D * VC; e += 256) {
        const int r = e / VC, c = e % VC;
        st.z[c][r] = Zs[(size_t)r * D + v0 + c];
        st.s[c][r] = Ss[(size_t)r * D + v0 + c];
      }
      __syncthreads();
#pragma unroll 4
      for (int c = 0; c < VC; ++c) {
        float zi[CPT], sj[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) zi[i] = st.z[c][grp + 16 * i];
#pragma unroll
        for (int j = 0; j < CPT; ++j) sj[j] = st.s[c][sub + 16 * j];
#pragma unroll
        for (int i = 0; i < CPT; ++i)
#pragma unroll
          for (int j = 0; j < CPT; ++j) acc[i][j] = fmaf(zi[i], sj[j], acc[i][j]);
      }
    }
  }
}

// Generic kernel (any D, fp32 or bf16 storage): dA_sym and dW in LDS with
// pitch D + 1; thread (grp, sub) takes token grp of a 16-token tile and the
// columns sub + 16 j.
template <typename T, int D>
__global__ __launch_bounds__(256) void vda_bwd_token_kernel(VdaBwdArgs<T> a) {
  constexpr int CPT = D / 16, TOK = 16, MP = D + 1;
  __shared__ float Am[D * MP];
  __shared__ float Wm[D * MP];
  struct KV { float k[TOK][MP]; float v[TOK][MP]; float b[TOK]; };
  __shared__ union { ZSStage<D> zs; KV kv; } u;

  const Geometry& g = a.g;
  const int nfr = g.F + (g.T > 0 ? 1 : 0);
  const int f = blockIdx.x % nfr;
  const int bh = blockIdx.x / nfr;
  const int tid = threadIdx.x, grp = tid >> 4, sub = tid & 15;
  const FrameTok<T> ft = frame_tok<T, D>(a, bh, f);
  if (!ft.text) alpha_scan_term<T, D>(a, ft, bh, f);
  if (ft.anchor) {                                   // no write: zero gradients
    zero_tokens(ft, D);
    return;
  }
  float acc[CPT][CPT];
  frame_zst<D>(ft.Z0, ft.S0, ft.Z1, ft.S1, u.zs, acc);
#pragma unroll
  for (int i = 0; i < CPT; ++i)
#pragma unroll
    for (int j = 0; j < CPT; ++j) Am[(grp + 16 * i) * MP + sub + 16 * j] = -acc[i][j];
  for (int e = tid; e < D * D; e += 256) {
    const int r = e / D, c = e % D;
    Wm[r * MP + c] = ft.Z0[e] + (ft.Z1 ? ft.Z1[e] : 0.f);
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
  for (long long n0 = 0; n0 < ft.ntok; n0 += TOK) {
    __syncthreads();
    for (int e = tid; e < TOK * D; e += 256) {
      const int r = e / D, c = e % D;
      const bool ok = n0 + r < ft.ntok;
      u.kv.k[r][c] = ok ? Elem<T>::load(ft.kp, (size_t)(n0 + r) * D + c) : 0.f;
      u.kv.v[r][c] = ok ? Elem<T>::load(ft.vp, (size_t)(n0 + r) * D + c) : 0.f;
    }
    if (tid < TOK) u.kv.b[tid] = n0 + tid < ft.ntok ? ft.bp[n0 + tid] : 0.f;
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
    if (n < ft.ntok) {
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int c = sub + 16 * j;
        Elem<T>::store(ft.dkp, (size_t)n * D + c, b * (E[j] + Gm[j]));
        Elem<T>::store(ft.dvp, (size_t)n * D + c, b * Fm[j]);
      }
      if (sub == 0) ft.dbp[n] = db;
    }
  }
}

// bf16 kernel (D = 64, 128) on v_mfma_f32_32x32x16_bf16.  NW waves; wave w
// owns the 32-channel block cb = w % (D/32) and the 32-token sub-tile
// w / (D/32) of each 64-token step.  dA_sym and dW are formed once per frame
// into LDS as bf16 hi + lo, row-major: the wave reads its rows of dA_sym and
// dW as A operands and its rows of dW^T through the transposing read, so no
// fragments stay in registers for the frame.  K and V rows come straight from
// global memory as B operands, the next step's while the current one is
// multiplied.  Per token (column n) and channel c:
//   acc1 = (dA_sym k + dW v)[c],  acc2 = (dW^T k)[c],
//   dk = beta acc1,  dv = beta acc2,  dbeta = 1/2 (acc1 . k + acc2 . v)
// (the last since k dW v = v dW^T k).
template <int D>
__global__ __launch_bounds__(BwdReadoutShape<D>::NW * 64) void vda_bwd_token_mfma_kernel(VdaBwdArgs<bf16_t> a) {
  constexpr int NB = D / 32, NKK = D / 16, NW = BwdReadoutShape<D>::NW, NT = NW * 64;
  constexpr int SUBT = NW / NB, TPS = 32 * SUBT;   // token sub-tiles and tokens per step
  constexpr int MP = D + 1, DP = D == 128 ? 152 : 72;   // DP: as in the readout adjoint
  // region 0 holds dA (fp32) until dA_sym is formed, then dW hi + lo;
  // region 1 holds dA_sym hi + lo
  struct DaF32 {
    float am[D * MP];
  };
  struct WHiLo {
    bf16_t wh[D * DP];
    bf16_t wl[D * DP];
  };
  __shared__ __attribute__((aligned(16))) union {
    DaF32 f;
    WHiLo w;
  } r0;
  __shared__ __attribute__((aligned(16))) struct {
    bf16_t sh[D * DP];
    bf16_t sl[D * DP];
  } r1;
  __shared__ float red[2][NW][32];

  const Geometry& g = a.g;
  const int nfr = g.F + (g.T > 0 ? 1 : 0);
  const int f = blockIdx.x % nfr;
  const int bh = blockIdx.x / nfr;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hg = lane >> 5, l32 = lane & 31;
  const int grp = lane >> 4, sl = lane & 15;       // 16-lane group of the transposing reads
  const FrameTok<bf16_t> ft = frame_tok<bf16_t, D>(a, bh, f);
  // the scan's alpha term and the anchor frames' zeros take the first 256
  // threads (whole waves)
  if (!ft.text && tid < 256) alpha_scan_term<bf16_t, D>(a, ft, bh, f);
  if (ft.anchor) {
    if (tid < 256) zero_tokens(ft, D);
    return;
  }
  {
    // dA = -(Z0 S0^T + Z1 S1^T) on v_mfma_f32_32x32x2f32, operands straight
    // from memory: rows of Z (A) and of S (B), 4 consecutive columns per
    // lane half and load.  Wave w computes the 32 x 32 blocks w + NW b.
    constexpr int NGB = NB * NB / NW, NK8 = D / 8;
    static_assert(NGB * NW == NB * NB, "dA blocks");
    f32x16 acc[NGB];
#pragma unroll
    for (int b = 0; b < NGB; ++b) acc[b] = f32x16{};
    for (int src = 0; src < (ft.Z1 ? 2 : 1); ++src) {
      const float* Zs = src ? ft.Z1 : ft.Z0;
      const float* Ss = src ? ft.S1 : ft.S0;
#pragma unroll 2
      for (int j = 0; j < NK8; ++j) {
        const int v0 = 8 * j + 4 * hg;
#pragma unroll
        for (int b = 0; b < NGB; ++b) {
          const int blk = wave + NW * b, ib = blk / NB, jb = blk % NB;
          const f32x4 za = *reinterpret_cast<const f32x4*>(Zs + (size_t)(ib * 32 + l32) * D + v0);
          const f32x4 sb = *reinterpret_cast<const f32x4*>(Ss + (size_t)(jb * 32 + l32) * D + v0);
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[b] = mfma32x32x2f32(za[q], sb[q], acc[b]);
        }
      }
    }
#pragma unroll
    for (int b = 0; b < NGB; ++b) {
      const int blk = wave + NW * b, ib = blk / NB, jb = blk % NB;
#pragma unroll
      for (int i = 0; i < 16; ++i) r0.f.am[(ib * 32 + mfma32_row(i, hg)) * MP + jb * 32 + l32] = -acc[b][i];
    }
  }
  __syncthreads();
  // dA_sym = dA + dA^T -> region 1 as bf16 hi + lo, four columns per item
  for (int e = tid; e < D * D / 4; e += NT) {
    const int c = e / (D / 4), k0 = (e % (D / 4)) * 4;
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2) {
      const int k = k0 + 2 * p2;
      const float x0 = r0.f.am[c * MP + k] + r0.f.am[k * MP + c];
      const float x1 = r0.f.am[c * MP + k + 1] + r0.f.am[(k + 1) * MP + c];
      const float h0 = bf16_to_f32(f32_to_bf16(x0)), h1 = bf16_to_f32(f32_to_bf16(x1));
      hw[p2] = pack_bf16x2(h0, h1);
      lw[p2] = pack_bf16x2(x0 - h0, x1 - h1);
    }
    *reinterpret_cast<u32x2*>(&r1.sh[c * DP + k0]) = u32x2{hw[0], hw[1]};
    *reinterpret_cast<u32x2*>(&r1.sl[c * DP + k0]) = u32x2{lw[0], lw[1]};
  }
  __syncthreads();      // dA is read out before dW takes its space
  // dW = Z0 + Z1 -> region 0 as bf16 hi + lo
  for (int e = tid; e < D * D / 4; e += NT) {
    const int c = e / (D / 4), k0 = (e % (D / 4)) * 4;
    f32x4 z = *reinterpret_cast<const f32x4*>(ft.Z0 + (size_t)c * D + k0);
    if (ft.Z1) {   // the text frame has one adjoint
      const f32x4 z1 = *reinterpret_cast<const f32x4*>(ft.Z1 + (size_t)c * D + k0);
#pragma unroll
      for (int j = 0; j < 4; ++j) z[j] = z[j] + z1[j];
    }
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int p2 = 0; p2 < 2; ++p2) {
      const float h0 = bf16_to_f32(f32_to_bf16(z[2 * p2])), h1 = bf16_to_f32(f32_to_bf16(z[2 * p2 + 1]));
      hw[p2] = pack_bf16x2(h0, h1);
      lw[p2] = pack_bf16x2(z[2 * p2] - h0, z[2 * p2 + 1] - h1);
    }
    *reinterpret_cast<u32x2*>(&r0.w.wh[c * DP + k0]) = u32x2{hw[0], hw[1]};
    *reinterpret_cast<u32x2*>(&r0.w.wl[c * DP + k0]) = u32x2{lw[0], lw[1]};
  }
  __syncthreads();
  const int cb = wave % NB, ts = wave / NB;
  const int c = cb * 32 + l32;
  // transposing reads of dW^T rows c: group lane sl points at row
  // k = 16 kk + 8 (grp / 2) + sl / 4 (+ 4), columns 32 cb + 16 (grp % 2) + 4 (sl % 4)
  const int wt_off = (8 * (grp >> 1) + (sl >> 2)) * DP + cb * 32 + 16 * (grp & 1) + 4 * (sl & 3);

  const long long ntok = ft.ntok;
  bf16x8 bk[NKK], bv[NKK], bkn[NKK], bvn[NKK];
  auto load_b = [&](long long n, bf16x8* dk_, bf16x8* dv_) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
      if (n < ntok) {
        x = ld16(ft.kp + (size_t)n * D + kk * 16 + hg * 8);
        y = ld16(ft.vp + (size_t)n * D + kk * 16 + hg * 8);
      }
      dk_[kk] = as_bf16x8(x);
      dv_[kk] = as_bf16x8(y);
    }
  };
  load_b(ts * 32 + l32, bk, bv);
  int it = 0;
  for (long long n0 = 0; n0 < ntok; n0 += TPS, ++it) {
    const long long n = n0 + ts * 32 + l32;
    load_b(n + TPS, bkn, bvn);
    f32x16 acc1 = f32x16{}, acc2 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int ao = c * DP + kk * 16 + hg * 8;
      const bf16x8 ash = as_bf16x8(ld16(&r1.sh[ao])), asl = as_bf16x8(ld16(&r1.sl[ao]));
      const bf16x8 wh = as_bf16x8(ld16(&r0.w.wh[ao])), wl = as_bf16x8(ld16(&r0.w.wl[ao]));
      const bf16_t* pth = &r0.w.wh[kk * 16 * DP + wt_off];
      const bf16_t* ptl = &r0.w.wl[kk * 16 * DP + wt_off];
      const u32x2 th0 = lds_read_tr16(pth), th1 = lds_read_tr16(pth + 4 * DP);
      const u32x2 tl0 = lds_read_tr16(ptl), tl1 = lds_read_tr16(ptl + 4 * DP);
      acc1 = mfma32x32x16(ash, bk[kk], acc1);
      acc1 = mfma32x32x16(asl, bk[kk], acc1);
      acc1 = mfma32x32x16(wh, bv[kk], acc1);
      acc1 = mfma32x32x16(wl, bv[kk], acc1);
      acc2 = mfma32x32x16(as_bf16x8(u32x4{th0[0], th0[1], th1[0], th1[1]}), bk[kk], acc2);
      acc2 = mfma32x32x16(as_bf16x8(u32x4{tl0[0], tl0[1], tl1[0], tl1[1]}), bk[kk], acc2);
    }
    const bool valid = n < ntok;
    // k and v at the accumulator positions (channels cb*32 + 8 i4 + 4 hg + r)
    // come from the step's B fragments: k-steps 2 cb and 2 cb + 1 hold them,
    // half in this lane and half in its partner (lane ^ 32); one
    // v_permlane32_swap per fragment word exchanges them.
    float kc[16], vc[16];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if ((kk >> 1) != cb) continue;       // wave-uniform: keeps the register index static
      const int m = kk & 1;
      const u32x4 wk = __builtin_bit_cast(u32x4, bk[kk]);
      const u32x4 wv = __builtin_bit_cast(u32x4, bv[kk]);
      uint32_t ok[4], pk_[4], ov[4], pv_[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const auto rk = __builtin_amdgcn_permlane32_swap(wk[w], wk[w], false, false);
        const auto rv = __builtin_amdgcn_permlane32_swap(wv[w], wv[w], false, false);
        ok[w] = hg ? rk[1] : rk[0];          // own word
        pk_[w] = hg ? rk[0] : rk[1];         // the partner's
        ov[w] = hg ? rv[1] : rv[0];
        pv_[w] = hg ? rv[0] : rv[1];
      }
#pragma unroll
      for (int odd = 0; odd < 2; ++odd) {
        const int i4 = 2 * m + odd;
        const bool own = hg == odd;
        // words 0,1 (lower half's slots 0..3) for hg = 0, words 2,3 for hg = 1
        const uint32_t k0w = own ? (hg ? ok[2] : ok[0]) : (hg ? pk_[2] : pk_[0]);
        const uint32_t k1w = own ? (hg ? ok[3] : ok[1]) : (hg ? pk_[3] : pk_[1]);
        const uint32_t v0w = own ? (hg ? ov[2] : ov[0]) : (hg ? pv_[2] : pv_[0]);
        const uint32_t v1w = own ? (hg ? ov[3] : ov[1]) : (hg ? pv_[3] : pv_[1]);
        kc[4 * i4 + 0] = bf16_to_f32((bf16_t)(k0w & 0xFFFFu));
        kc[4 * i4 + 1] = bf16_to_f32((bf16_t)(k0w >> 16));
        kc[4 * i4 + 2] = bf16_to_f32((bf16_t)(k1w & 0xFFFFu));
        kc[4 * i4 + 3] = bf16_to_f32((bf16_t)(k1w >> 16));
        vc[4 * i4 + 0] = bf16_to_f32((bf16_t)(v0w & 0xFFFFu));
        vc[4 * i4 + 1] = bf16_to_f32((bf16_t)(v0w >> 16));
        vc[4 * i4 + 2] = bf16_to_f32((bf16_t)(v1w & 0xFFFFu));
        vc[4 * i4 + 3] = bf16_to_f32((bf16_t)(v1w >> 16));
      }
    }
    float db = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      db = fmaf(acc1[i], kc[i], db);
      db = fmaf(acc2[i], vc[i], db);
    }
    if (valid) {
      const float b = ft.bp[n];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int c0 = cb * 32 + 8 * i4 + 4 * hg;
        u32x2 pk, pv;
        pk[0] = pack_bf16x2(b * acc1[4 * i4 + 0], b * acc1[4 * i4 + 1]);
        pk[1] = pack_bf16x2(b * acc1[4 * i4 + 2], b * acc1[4 * i4 + 3]);
        pv[0] = pack_bf16x2(b * acc2[4 * i4 + 0], b * acc2[4 * i4 + 1]);
        pv[1] = pack_bf16x2(b * acc2[4 * i4 + 2], b * acc2[4 * i4 + 3]);
        *reinterpret_cast<u32x2*>(ft.dkp + (size_t)n * D + c0) = pk;
        *reinterpret_cast<u32x2*>(ft.dvp + (size_t)n * D + c0) = pv;
      }
    }
    db = half_sum(db);
    if (hg == 0) red[it & 1][wave][l32] = db;
    lds_barrier();
    if (cb == 0 && hg == 0 && valid) {
      float s = 0.f;
#pragma unroll
      for (int b2 = 0; b2 < NB; ++b2) s += red[it & 1][ts * NB + b2][l32];
      ft.dbp[n] = 0.5f * s;
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      bk[kk] = bkn[kk];
      bv[kk] = bvn[kk];
    }
  }
}

// 8. dgamma = sum of the per-(b, h, frame) partial sums: one workgroup per
//    channel, a fixed-order tree over the rows.
__global__ __launch_bounds__(256) void vda_bwd_dgamma_kernel(const float* __restrict__ dgp, long long rows,
                                                             int D, float* __restrict__ dgamma) {
  __shared__ float part[256];
  const int c = blockIdx.x;
  float s = 0.f;
  for (long long r = threadIdx.x; r < rows; r += 256) s += dgp[r * D + c];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) dgamma[c] = part[0];
}

template <typename T, int D>
hipError_t launch_all(const VdaBwdArgs<T>& a, const float* Tf, const float* Uf, float* dgamma,
                      int stage, hipStream_t s) {
  const Geometry& g = a.g;
  const unsigned BH = (unsigned)(g.B * g.H);
  constexpr int NCB = (D + kBCB - 1) / kBCB;
  if (stage == 0) {
    if constexpr (std::is_same<T, bf16_t>::value && (D == 64 || D == 128))
      vda_bwd_readout_mfma_kernel<D><<<BH * g.F, BwdReadoutShape<D>::NW * 64, 0, s>>>(a);
    else
      vda_bwd_readout_kernel<T, D><<<BH * g.F, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  vda_bwd_dp_kernel<T, D><<<BH * 2 * (g.C + 1), 256, 0, s>>>(a);
  vda_bwd_alpha_bridge_kernel<T, D><<<BH * (D / kBridgeCh), 64,
                                      ((size_t)5 * g.F * kBridgeCh + 2 * g.F + 2 * g.C + 1) * 4, s>>>(a);
  if constexpr (D == 64 || D == 128)
    vda_bwd_chunk_adjoint_mfma_kernel<T, D><<<BH * 2 * NCB, 256, 0, s>>>(a);
  else
    vda_bwd_chunk_adjoint_kernel<T, D><<<BH * 2 * NCB, 256, 0, s>>>(a);
  if (g.T > 0) vda_bwd_text_kernel<T, D><<<BH * NCB, 256, 0, s>>>(a);
  if constexpr (D == 64 || D == 128)
    vda_bwd_frame_adjoint_mfma_kernel<T, D><<<BH * 2 * g.C * NCB, 256, 0, s>>>(a, Tf, Uf);
  else
    vda_bwd_frame_adjoint_kernel<T, D><<<BH * 2 * g.C * NCB, 256, 0, s>>>(a, Tf, Uf);
  const unsigned nfr = BH * (g.F + (g.T > 0 ? 1 : 0));
  if constexpr (std::is_same<T, bf16_t>::value && (D == 64 || D == 128))
    vda_bwd_token_mfma_kernel<D><<<nfr, BwdReadoutShape<D>::NW * 64, 0, s>>>(a);
  else
    vda_bwd_token_kernel<T, D><<<nfr, 256, 0, s>>>(a);
  if (dgamma && a.dgp) vda_bwd_dgamma_kernel<<<D, 256, 0, s>>>(a.dgp, (long long)BH * g.F, D, dgamma);
  return hipGetLastError();
}

}  // namespace

template <typename T>
hipError_t launch_vda_bwd(const Geometry& g, const VdaBwdPtrs& p, const T* q, const T* k, const T* v,
                          const T* k_text, const T* v_text, const T* d_out, T* dq, T* dk, T* dv,
                          T* dk_text, T* dv_text, float eps, float init_scale, int stage,
                          hipStream_t s) {
  VdaBwdArgs<T> a{g, q, k, v, p.beta, p.alpha, k_text, v_text, p.beta_text, p.g_l, p.gamma, d_out,
                  eps, init_scale, p.Pf, p.Pr, p.St, p.Xf, p.Tc, p.G, p.Dbr, p.dDbr,
                  p.dgamma ? p.dgp : nullptr, p.dP, p.mu, p.Sst, p.Zst, p.ZT, p.Rscr, dq, dk, dv,
                  p.dbeta, p.dalpha, dk_text, dv_text, p.dbeta_text, p.dg_l};
  switch (g.D) {
    case 16: return launch_all<T, 16>(a, p.Tf, p.Uf, p.dgamma, stage, s);
    case 32: return launch_all<T, 32>(a, p.Tf, p.Uf, p.dgamma, stage, s);
    case 64: return launch_all<T, 64>(a, p.Tf, p.Uf, p.dgamma, stage, s);
    case 128: return launch_all<T, 128>(a, p.Tf, p.Uf, p.dgamma, stage, s);
    default: return hipErrorInvalidValue;
  }
}

template hipError_t launch_vda_bwd<float>(const Geometry&, const VdaBwdPtrs&, const float*, const float*,
                                          const float*, const float*, const float*, const float*,
                                          float*, float*, float*, float*, float*, float, float,
                                          int, hipStream_t);
template hipError_t launch_vda_bwd<bf16_t>(const Geometry&, const VdaBwdPtrs&, const bf16_t*,
                                           const bf16_t*, const bf16_t*, const bf16_t*, const bf16_t*,
                                           const bf16_t*, bf16_t*, bf16_t*, bf16_t*, bf16_t*, bf16_t*,
                                           float, float, int, hipStream_t);

}  // namespace vdn
