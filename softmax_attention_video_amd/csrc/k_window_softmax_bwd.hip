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
// dK and dV together.  Visibility is symmetric, so the forward's items read with the
// roles swapped (the group's frames as keys, its spans as the queries that
// see them) cover every (query, key) pair exactly once, and every output row
// is written by one workgroup: no atomics.
//
// Text keys (method, bidirectional linear attention: the text stays visible
// to the Softmax branch): the T text tokens are keys of every query in the
// same softmax.  The query-stationary pass walks them as one more key span;
// the key-stationary pass gets extra items, blocks of text keys whose query
// span is the whole video.
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

// Key-stationary work items of the text keys: blocks of bk text keys, each
// seen by every video query ([0, L) as one span).  They lead the grid (as
// long as the anchor items, so they start first), padded to a multiple of
// the XCD count so the video items keep their XCD placement.
__host__ __device__ inline int text_key_blocks(const Geometry& g, int bk) {
  return g.Ts > 0 ? g.B * g.H * ((g.Ts + bk - 1) / bk) : 0;
}
__host__ __device__ inline int text_items_padded(const Geometry& g, int bk) {
  return (text_key_blocks(g, bk) + kNumXcd - 1) / kNumXcd * kNumXcd;
}
// Decodes workgroup bid of a key-stationary kernel whose first ntext
// workgroups take text key blocks; text: the item's keys are text keys
// (key range [k0, Ts) of it.q_begin .. it.q_end).
__device__ __forceinline__ bool decode_key_item(const Geometry& g, const SoftmaxWork& w, int bk,
                                                int ntext, int bid, Item& it, int& k0, bool& text) {
  text = bid < ntext;
  if (!text) return decode_item<false>(g, w, bk, bid - ntext, 0, it, k0);
  const int nb = (g.Ts + bk - 1) / bk;
  if (bid >= g.B * g.H * nb) return false;
  it.bh = bid / nb;
  k0 = (bid % nb) * bk;
  it.q_begin = 0;
  it.q_end = g.Ts;
  it.nspan = 1;
  it.kb0 = 0;
  it.ke0 = (int)g.L;
  it.kb1 = it.ke1 = it.kb2 = it.ke2 = it.kb3 = it.ke3 = 0;
  return true;
}

// ---------------------------------------------------------------------------
// Generic SIMT kernels (fp32 or bf16 storage, any D <= 128, any N).
// dQ: one thread per query, key tiles of 32 staged through LDS.
// ---------------------------------------------------------------------------
template <typename T, int DMAX>
__global__ __launch_bounds__(128) void softmax_bwd_dq_simt_kernel(
    Geometry g, SoftmaxWork w, const T* __restrict__ qp, const T* __restrict__ kp,
    const T* __restrict__ vp, const T* __restrict__ ktp, const T* __restrict__ vtp,
    const T* __restrict__ dop, const float* __restrict__ lse, const float* __restrict__ Dq,
    T* __restrict__ dq, float scale) {
  constexpr int BQ = 128, BK = 32;
  __shared__ float Ks[BK][DMAX + 1];
  __shared__ float Vs[BK][DMAX + 1];
  Item it;
  int q0;
  // text keys (g.Ts > 0) are a fourth span, walk positions L .. L + Ts - 1
  if (!decode_item<true>(g, w, BQ, blockIdx.x, g.Ts, it, q0)) return;
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
  const SpanWalk<BK, 4> walk(it);
  for (int jt = 0; jt < walk.n; ++jt) {
    int ks, nk;
    walk.tile(jt, ks, nk);
    const bool tx = ks >= L;
    const T* kb = tx ? ktp : kp;
    const T* vb = tx ? vtp : vp;
    const size_t kbase = tx ? ((size_t)it.bh * g.Ts + (ks - L)) * D : base + (size_t)ks * D;
    __syncthreads();
    for (int e = threadIdx.x; e < BK * D; e += blockDim.x) {
      const int r = e / D, c = e % D;
      Ks[r][c] = r < nk ? Elem<T>::load(kb, kbase + (size_t)r * D + c) : 0.f;
      Vs[r][c] = r < nk ? Elem<T>::load(vb, kbase + (size_t)r * D + c) : 0.f;
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
    Geometry g, SoftmaxWork w, int ntext, const T* __restrict__ qp, const T* __restrict__ kp,
    const T* __restrict__ vp, const T* __restrict__ ktp, const T* __restrict__ vtp,
    const T* __restrict__ dop, const float* __restrict__ lse, const float* __restrict__ Dq,
    T* __restrict__ dk, T* __restrict__ dv, T* __restrict__ dkt, T* __restrict__ dvt,
    float scale) {
  constexpr int BK = 128, BQ = 32;
  __shared__ float Qs[BQ][DMAX + 1];
  __shared__ float Ds[BQ][DMAX + 1];
  __shared__ float Ls[BQ], Dd[BQ];
  Item it;
  int k0;
  bool text;
  if (!decode_key_item(g, w, BK, ntext, blockIdx.x, it, k0, text)) return;
  const int D = g.D;
  const long long L = g.L;
  const int krow = k0 + threadIdx.x;
  const bool kvalid = krow < it.q_end;
  const size_t base = (size_t)it.bh * L * D;
  // the item's keys: video rows of this head, or its text keys
  const size_t kbase = text ? (size_t)it.bh * g.Ts * D : base;
  const T* kb = text ? ktp : kp;
  const T* vb = text ? vtp : vp;
  T* dkb = text ? dkt : dk;
  T* dvb = text ? dvt : dv;
  float kv[DMAX], vv[DMAX], ak[DMAX], av[DMAX];
#pragma unroll
  for (int j = 0; j < DMAX; ++j) {
    kv[j] = (j < D && kvalid) ? Elem<T>::load(kb, kbase + (size_t)krow * D + j) : 0.f;
    vv[j] = (j < D && kvalid) ? Elem<T>::load(vb, kbase + (size_t)krow * D + j) : 0.f;
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
      Elem<T>::store(dkb, kbase + (size_t)krow * D + j, ak[j] * scale);
      Elem<T>::store(dvb, kbase + (size_t)krow * D + j, av[j]);
    }
}

template <typename T>
hipError_t launch_softmax_bwd_simt(const Geometry& g, const T* q, const T* k, const T* v,
                                   const T* do_hm, const float* lse, const float* Dq, T* dq, T* dk,
                                   T* dv, const SoftmaxBwdText& tx, float scale, hipStream_t s) {
  if (g.Ts > 0 && (!tx.k_text || !tx.v_text || !tx.dk_text || !tx.dv_text)) return hipErrorInvalidValue;
  const SoftmaxWork wq = window_work(g, 128);
  const SoftmaxWork wk = window_work(g, 128);
  if (wq.grid == 0) return hipSuccess;
  const int ntext = text_items_padded(g, 128);
  const T* kt = (const T*)tx.k_text;
  const T* vt = (const T*)tx.v_text;
  T* dkt = (T*)tx.dk_text;
  T* dvt = (T*)tx.dv_text;
#define VDN_BWD_SIMT(DM)                                                                           \
  softmax_bwd_dq_simt_kernel<T, DM><<<wq.grid, 128, 0, s>>>(g, wq, q, k, v, kt, vt, do_hm, lse, Dq, dq, scale); \
  softmax_bwd_dkdv_simt_kernel<T, DM><<<ntext + wk.grid, 128, 0, s>>>(g, wk, ntext, q, k, v, kt, vt, do_hm, lse, Dq, dk, dv, dkt, dvt, scale)
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

// ---------------------------------------------------------------------------
// bf16 MFMA kernels (D = 64, 128; N % 16 == 0) with fp32 accumulation: dQ on
// v_mfma_f32_32x32x16_bf16, dK and dV on v_mfma_f32_16x16x32_bf16 (below).
// Tiles are staged global -> registers -> LDS one tile
// ahead with one workgroup barrier per tile; rows past a span's end read as
// zero through the buffer descriptors.
//
// dQ (query-stationary, 8 waves x 32 queries): per 32-key block
//   S^T  = K Q^T        (A: K rows from LDS, B: the wave's Q fragments)
//   dP^T = V dO^T       (A: V rows from LDS, B: the wave's dO fragments)
//   dS^T = P^T (dP^T - Dq),  P^T = exp2(S^T scale log2e - lse log2e)
//   dQ^T += K^T dS^T    (A: K^T rows from LDS, B: dS^T from registers)
// K rows are loaded in key_perm order so a lane half holds 16 consecutive
// keys of the block in register order, which is the B layout of the last
// product; lse and Dq are per lane (one query per lane).
// ---------------------------------------------------------------------------
struct BwdArgs {
  Geometry g;
  SoftmaxWork w;
  const bf16_t* q;      // [B,H,L,D]
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* dO;     // g_s * dOhat, [B,H,L,D]
  const bf16_t* kt;     // K^T  [B,H,D,L]
  const bf16_t* qt;     // Q^T  [B,H,D,L]
  const bf16_t* dOt;    // dO^T [B,H,D,L]
  const float* lse;     // [B,H,L], natural log
  const float* Dq;      // [B,H,L]
  bf16_t* dq;
  bf16_t* dk;
  bf16_t* dv;
  // text keys (g.Ts > 0): k_text, v_text [B,H,Ts,D], their transpose
  // [B,H,D,Tp] (Tp = Ts rounded up to 16, zero columns past Ts) and the
  // gradients dk_text, dv_text [B,H,Ts,D]
  const bf16_t* k_text;
  const bf16_t* v_text;
  const bf16_t* ktt;
  bf16_t* dk_text;
  bf16_t* dv_text;
  int tpitch;           // Tp
  int ntext;            // leading workgroups of the dK/dV kernel that take text keys
  float scale, scale_log2;
};



constexpr int kBwdQW = 8;          // dQ kernel: waves (32 queries each)
constexpr int kBwdBK = 64;         // keys per staged tile (dQ) / queries per staged tile (dK, dV)

template <int D, bool TEXT>
__global__ __launch_bounds__(kBwdQW * 64) void softmax_bwd_dq_mfma_kernel(BwdArgs a) {
  constexpr int NT = kBwdQW * 64, BQ = kBwdQW * 32, BK = kBwdBK;
  constexpr int KP = D + 8, TP = BK + 8;
  constexpr int NKK = D / 16, NDB = D / 32, NB = BK / 32;
  constexpr int RCH = BK * D / 8 / NT, TCH = D * BK / 8 / NT;   // 16-byte chunks per thread
  static_assert(RCH * NT * 8 == BK * D && TCH * NT * 8 == D * BK, "tile split");
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][BK * KP];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][BK * KP];
  __shared__ __attribute__((aligned(16))) bf16_t Kts[2][D * TP];
  const Geometry& g = a.g;
  Item it;
  int q0;
  if (!decode_item<TEXT>(g, a.w, BQ, blockIdx.x, TEXT ? g.Ts : 0, it, q0)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hg = lane >> 5, l32 = lane & 31;
  const long long L = g.L;
  const size_t hb = (size_t)it.bh * L * D;
  const bf16_t* K = a.k + hb;
  const bf16_t* V = a.v + hb;
  const bf16_t* Kt = a.kt + hb;
  // text keys (walk positions from L on)
  const size_t hbt = TEXT ? (size_t)it.bh * g.Ts * D : 0;
  const bf16_t* KT = TEXT ? a.k_text + hbt : nullptr;
  const bf16_t* VT = TEXT ? a.v_text + hbt : nullptr;
  const bf16_t* KTt = TEXT ? a.ktt + (size_t)it.bh * D * a.tpitch : nullptr;
  const int qrow = q0 + wave * 32 + l32;
  const bool qvalid = qrow < it.q_end;
  bf16x8 qf[NKK], df[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    if (qvalid) {
      x = ld16(a.q + hb + (size_t)qrow * D + kk * 16 + hg * 8);
      y = ld16(a.dO + hb + (size_t)qrow * D + kk * 16 + hg * 8);
    }
    qf[kk] = as_bf16x8(x);
    df[kk] = as_bf16x8(y);
  }
  const float lse2 = qvalid ? a.lse[(size_t)it.bh * L + qrow] * kLog2e : 0.f;
  const float dqv = qvalid ? a.Dq[(size_t)it.bh * L + qrow] : 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) acc[b] = f32x16{};
  const SpanWalk<BK, TEXT ? 4 : 3> walk(it);
  const uint32_t kt_bytes = (uint32_t)min((long long)D * L * 2, 0x7FFFFFF0ll);
  u32x4 cr[2 * RCH + TCH];
  auto load_tile = [&](int j) {
    int ks, nk;
    walk.tile(j, ks, nk);
    const bool tx = TEXT && ks >= L;
    const int kr = tx ? ks - (int)L : ks;                // row in its own key array
    const long long pitch = tx ? a.tpitch : L;           // row pitch of the transposed keys
    const rsrc_t rk = make_rsrc((tx ? KT : K) + (size_t)kr * D, (uint32_t)nk * D * 2);
    const rsrc_t rv = make_rsrc((tx ? VT : V) + (size_t)kr * D, (uint32_t)nk * D * 2);
    const rsrc_t rt = tx ? make_rsrc(KTt + kr, (uint32_t)(D * pitch - kr) * 2)
                         : make_rsrc(Kt + ks, kt_bytes - (uint32_t)ks * 2);
#pragma unroll
    for (int i = 0; i < RCH; ++i) {
      const int c = tid + NT * i;
      const uint32_t off = (uint32_t)((c / (D / 8)) * D + (c % (D / 8)) * 8) * 2;
      cr[i] = buf_ld16(rk, off);
      cr[RCH + i] = buf_ld16(rv, off);
    }
#pragma unroll
    for (int i = 0; i < TCH; ++i) {
      const int c = tid + NT * i;
      const int r = c / (BK / 8), c8 = c % (BK / 8);
      cr[2 * RCH + i] = buf_ld16(rt, c8 * 8 < nk ? (uint32_t)(r * pitch + c8 * 8) * 2 : 0x80000000u);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RCH; ++i) {
      const int c = tid + NT * i;
      const int off = (c / (D / 8)) * KP + (c % (D / 8)) * 8;
      st16(&Ks[buf][off], cr[i]);
      st16(&Vs[buf][off], cr[RCH + i]);
    }
#pragma unroll
    for (int i = 0; i < TCH; ++i) {
      const int c = tid + NT * i;
      st16(&Kts[buf][(c / (BK / 8)) * TP + (c % (BK / 8)) * 8], cr[2 * RCH + i]);
    }
  };
  const int rperm = key_perm(l32);
  if (walk.n > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int j = 0; j < walk.n; ++j) {
    const int buf = j & 1;
    int ks, nk;
    walk.tile(j, ks, nk);
    if (j + 1 < walk.n) load_tile(j + 1);
    const bf16_t* Kb = Ks[buf];
    const bf16_t* Vb = Vs[buf];
    const bf16_t* Tb = Kts[buf];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      f32x16 s = {}, dp = {};
      const bf16_t* kr = Kb + (blk * 32 + rperm) * KP + hg * 8;
      const bf16_t* vr = Vb + (blk * 32 + rperm) * KP + hg * 8;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        s = mfma32x32x16(as_bf16x8(ld16(kr + kk * 16)), qf[kk], s);
        dp = mfma32x32x16(as_bf16x8(ld16(vr + kk * 16)), df[kk], dp);
      }
      // video spans hold whole 16-key groups; the text span may end inside one
      const bool valid = blk * 32 + hg * 16 < nk;
      bf16x8 pb[2];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const bool vk = TEXT ? blk * 32 + hg * 16 + i < nk : valid;
        const float p = vk ? fast_exp2(fmaf(s[i], a.scale_log2, -lse2)) : 0.f;
        pb[i >> 3][i & 7] = static_cast<__bf16>(p * (dp[i] - dqv));
      }
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int b = 0; b < NDB; ++b) {
          const bf16x8 kf = as_bf16x8(ld16(Tb + (b * 32 + l32) * TP + blk * 32 + hg * 16 + h2 * 8));
          acc[b] = mfma32x32x16(kf, pb[h2], acc[b]);
        }
    }
    if (j + 1 < walk.n) store_tile(buf ^ 1);
    __syncthreads();
  }
  if (!qvalid) return;
  bf16_t* orow = a.dq + hb + (size_t)qrow * D;
#pragma unroll
  for (int b = 0; b < NDB; ++b)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = b * 32 + 8 * i4 + 4 * hg;
      u32x2 pk;
      pk[0] = pack_bf16x2(acc[b][i4 * 4 + 0] * a.scale, acc[b][i4 * 4 + 1] * a.scale);
      pk[1] = pack_bf16x2(acc[b][i4 * 4 + 2] * a.scale, acc[b][i4 * 4 + 3] * a.scale);
      *reinterpret_cast<u32x2*>(orow + d) = pk;
    }
}

// v_mfma_f32_16x16x32_bf16 (wave64): lane l supplies row l % 16 of A and
// column l % 16 of B, each with contraction slots 8 (l / 16) .. 8 (l / 16) + 7;
// the 16 x 16 result holds column l % 16, rows 4 (l / 16) .. 4 (l / 16) + 3.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

constexpr int kBwdFW = 8;          // fused dK / dV kernel: waves, 16 keys each

// dK and dV together (key-stationary: the item's frames are the keys, its
// spans the queries that see them), one wave per 16 keys on
// 16 x 16 x 32 products, so that S and dP are formed once for both
// gradients (8 d flops per visible pair) and the wave's K and V fragments,
// S, dP and both accumulators fit two waves per SIMD.  Per 32-query block:
//   S  = Q K^T,  dP = dO V^T      (A: Q / dO rows from LDS, B: K / V fragments)
//   P = exp2(S scale log2e - lse log2e),  dS = P (dP - Dq)
//   dV^T += dO^T P,  dK^T += Q^T dS   (A: dO^T / Q^T rows from LDS, B: P / dS)
// A lane of S holds one key and the queries 16 r + 4 (l / 16) + i of row
// tile r = 0, 1; taken in that order as the eight contraction slots of the
// accumulation they are its B operand directly, and the transposed tiles are
// stored with each block's columns in the same order (two 8-byte pieces per
// staged 16-byte chunk), so the A operand is one 16-byte read per lane.
template <int D>
__global__ __launch_bounds__(kBwdFW * 64) void softmax_bwd_dkdv16_kernel(BwdArgs a) {
  constexpr int NT = kBwdFW * 64, BKEY = kBwdFW * 16, BQ = kBwdBK;
  // row pitches of 32 bytes times an odd number: the 32 lanes that one LDS
  // cycle serves (16 rows, two 16-byte column groups) then cover all banks
  constexpr int KP = D + 16, TP = BQ + 16;
  static_assert((KP * 2 / 32) % 2 == 1 && (TP * 2 / 32) % 2 == 1, "row pitch");
  constexpr int NKS = D / 32, NDT = D / 16, NB = BQ / 32;
  constexpr int RCH = BQ * D / 8 / NT, TCH = D * BQ / 8 / NT;
  static_assert(RCH * NT * 8 == BQ * D && TCH * NT * 8 == D * BQ, "tile split");
  static_assert(NB == 2, "two query blocks per tile");
  __shared__ __attribute__((aligned(16))) bf16_t Qs[2][BQ * KP];
  __shared__ __attribute__((aligned(16))) bf16_t Ds[2][BQ * KP];
  __shared__ __attribute__((aligned(16))) bf16_t Qt[2][D * TP];
  __shared__ __attribute__((aligned(16))) bf16_t Dt[2][D * TP];
  __shared__ __attribute__((aligned(16))) float Ls[2][BQ];
  __shared__ __attribute__((aligned(16))) float Dd[2][BQ];
  const Geometry& g = a.g;
  Item it;
  int k0;
  bool text;
  if (!decode_key_item(g, a.w, BKEY, a.ntext, blockIdx.x, it, k0, text)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4, l16 = lane & 15;
  const long long L = g.L;
  const size_t hb = (size_t)it.bh * L * D;
  // the item's keys: video rows of this head, or its text keys
  const size_t hk = text ? (size_t)it.bh * g.Ts * D : hb;
  const bf16_t* Kk = text ? a.k_text : a.k;
  const bf16_t* Vk = text ? a.v_text : a.v;
  bf16_t* dKk = text ? a.dk_text : a.dk;
  bf16_t* dVk = text ? a.dv_text : a.dv;
  const bf16_t* Q = a.q + hb;
  const bf16_t* dO = a.dO + hb;
  const bf16_t* QT = a.qt + hb;
  const bf16_t* dOT = a.dOt + hb;
  const float* lse = a.lse + (size_t)it.bh * L;
  const float* Dq = a.Dq + (size_t)it.bh * L;
  const int krow = k0 + wave * 16 + l16;
  const bool kvalid = krow < it.q_end;
  bf16x8 kf[NKS], vf[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    u32x4 x = {0, 0, 0, 0}, y = {0, 0, 0, 0};
    if (kvalid) {
      x = ld16(Kk + hk + (size_t)krow * D + ks * 32 + grp * 8);
      y = ld16(Vk + hk + (size_t)krow * D + ks * 32 + grp * 8);
    }
    kf[ks] = as_bf16x8(x);
    vf[ks] = as_bf16x8(y);
  }
  f32x4 accK[NDT], accV[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    accK[t] = f32x4{};
    accV[t] = f32x4{};
  }
  const SpanWalk<BQ, 3> walk(it);
  const uint32_t t_bytes = (uint32_t)min((long long)D * L * 2, 0x7FFFFFF0ll);
  u32x4 c0r[2 * RCH], c1r[2 * TCH];
  float cl = 0.f, cd = 0.f;
  auto load_piece0 = [&](int j) {      // Q and dO rows
    int qs, nq;
    walk.tile(j, qs, nq);
    const rsrc_t rq = make_rsrc(Q + (size_t)qs * D, (uint32_t)nq * D * 2);
    const rsrc_t rd = make_rsrc(dO + (size_t)qs * D, (uint32_t)nq * D * 2);
#pragma unroll
    for (int i = 0; i < RCH; ++i) {
      const int c = tid + NT * i;
      const uint32_t off = (uint32_t)((c / (D / 8)) * D + (c % (D / 8)) * 8) * 2;
      c0r[i] = buf_ld16(rq, off);
      c0r[RCH + i] = buf_ld16(rd, off);
    }
  };
  auto store_piece0 = [&](int buf) {
#pragma unroll
    for (int i = 0; i < RCH; ++i) {
      const int c = tid + NT * i;
      const int off = (c / (D / 8)) * KP + (c % (D / 8)) * 8;
      st16(&Qs[buf][off], c0r[i]);
      st16(&Ds[buf][off], c0r[RCH + i]);
    }
  };
  auto load_piece1 = [&](int j) {      // Q^T and dO^T, lse and Dq
    int qs, nq;
    walk.tile(j, qs, nq);
    const rsrc_t rt = make_rsrc(QT + qs, t_bytes - (uint32_t)qs * 2);
    const rsrc_t ru = make_rsrc(dOT + qs, t_bytes - (uint32_t)qs * 2);
#pragma unroll
    for (int i = 0; i < TCH; ++i) {
      const int c = tid + NT * i;
      const int r = c / (BQ / 8), c8 = c % (BQ / 8);
      const uint32_t off = c8 * 8 < nq ? (uint32_t)(r * L + c8 * 8) * 2 : 0x80000000u;
      c1r[i] = buf_ld16(rt, off);
      c1r[TCH + i] = buf_ld16(ru, off);
    }
    if (tid < BQ) {
      cl = tid < nq ? lse[qs + tid] * kLog2e : INFINITY;
      cd = tid < nq ? Dq[qs + tid] : 0.f;
    }
  };
  // a staged chunk holds queries 8 m .. 8 m + 7 of a block (m = 0..3); its
  // halves go to the slot positions 16 (m % 2) + 4 (m / 2) and that + 8
  auto store_piece1 = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TCH; ++i) {
      const int c = tid + NT * i;
      const int r = c / (BQ / 8), c8 = c % (BQ / 8), m = c8 & 3;
      const int p = r * TP + (c8 >> 2) * 32 + 16 * (m & 1) + 4 * (m >> 1);
      const u32x2 lo = {c1r[i][0], c1r[i][1]}, hi = {c1r[i][2], c1r[i][3]};
      *reinterpret_cast<u32x2*>(&Qt[buf][p]) = lo;
      *reinterpret_cast<u32x2*>(&Qt[buf][p + 8]) = hi;
      const u32x2 lo2 = {c1r[TCH + i][0], c1r[TCH + i][1]}, hi2 = {c1r[TCH + i][2], c1r[TCH + i][3]};
      *reinterpret_cast<u32x2*>(&Dt[buf][p]) = lo2;
      *reinterpret_cast<u32x2*>(&Dt[buf][p + 8]) = hi2;
    }
    if (tid < BQ) {
      Ls[buf][tid] = cl;
      Dd[buf][tid] = cd;
    }
  };
  // S and dP of query block qb: row tile r holds queries qb 32 + 16 r + ...
  auto sdp = [&](int buf, int qb, f32x4* sv, f32x4* dpv) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      sv[r] = f32x4{};
      dpv[r] = f32x4{};
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int off = (qb * 32 + r * 16 + l16) * KP + ks * 32 + grp * 8;
        sv[r] = mfma16x16x32(as_bf16x8(ld16(&Qs[buf][off])), kf[ks], sv[r]);
        dpv[r] = mfma16x16x32(as_bf16x8(ld16(&Ds[buf][off])), vf[ks], dpv[r]);
      }
  };
  // P and dS as bf16 operands, slot 4 r + i = query qb 32 + 16 r + 4 grp + i
  auto probs = [&](int buf, int qb, const f32x4* sv, const f32x4* dpv, bf16x8& pb, bf16x8& db) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int q = qb * 32 + 16 * r + 4 * grp;
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&Ls[buf][q]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Dd[buf][q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = fast_exp2(fmaf(sv[r][e], a.scale_log2, -l4[e]));
        pb[4 * r + e] = static_cast<__bf16>(pv);
        db[4 * r + e] = static_cast<__bf16>(pv * (dpv[r][e] - d4[e]));
      }
    }
  };
  auto accum = [&](int buf, int qb, const bf16x8& pb, const bf16x8& db) {
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      const int off = (16 * t + l16) * TP + qb * 32 + 8 * grp;
      accV[t] = mfma16x16x32(as_bf16x8(ld16(&Dt[buf][off])), pb, accV[t]);
      accK[t] = mfma16x16x32(as_bf16x8(ld16(&Qt[buf][off])), db, accK[t]);
    }
  };
  if (walk.n > 0) {
    load_piece0(0);
    load_piece1(0);
    store_piece0(0);
    store_piece1(0);
  }
  __syncthreads();
  for (int j = 0; j < walk.n; ++j) {
    const int buf = j & 1;
    // the next tile is requested now and stored at the end (into the buffer
    // the last barrier released); the last tile restages itself there, which
    // keeps the body one straight-line block for the issue order below
    const int jn = j + 1 < walk.n ? j + 1 : j;
    load_piece0(jn);
    load_piece1(jn);
    f32x4 s0[2], d0[2], s1[2], d1[2];
    bf16x8 p0, g0, p1, g1;
    sdp(buf, 0, s0, d0);
    sdp(buf, 1, s1, d1);
    probs(buf, 0, s0, d0, p0, g0);
    accum(buf, 0, p0, g0);
    probs(buf, 1, s1, d1, p1, g1);
    accum(buf, 1, p1, g1);
    store_piece0(buf ^ 1);
    store_piece1(buf ^ 1);
    // issue order: block 0's S and dP; block 1's among block 0's
    // probabilities; block 0's accumulation among block 1's probabilities;
    // block 1's accumulation
#pragma unroll
    for (int u = 0; u < 4 * NKS; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
#pragma unroll
    for (int u = 0; u < 4 * NKS; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
#pragma unroll
    for (int u = 0; u < 2 * NDT; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
#pragma unroll
    for (int u = 0; u < 2 * NDT; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __syncthreads();
  }
  if (!kvalid) return;
  bf16_t* krk = dKk + hk + (size_t)krow * D;
  bf16_t* krv = dVk + hk + (size_t)krow * D;
#pragma unroll
  for (int t = 0; t < NDT; ++t) {
    const int d = 16 * t + 4 * grp;
    u32x2 pk, pv;
    pk[0] = pack_bf16x2(accK[t][0] * a.scale, accK[t][1] * a.scale);
    pk[1] = pack_bf16x2(accK[t][2] * a.scale, accK[t][3] * a.scale);
    pv[0] = pack_bf16x2(accV[t][0], accV[t][1]);
    pv[1] = pack_bf16x2(accV[t][2], accV[t][3]);
    *reinterpret_cast<u32x2*>(krk + d) = pk;
    *reinterpret_cast<u32x2*>(krv + d) = pv;
  }
}

bool softmax_bwd_mfma_ok(const Geometry& g) {
  return (g.D == 64 || g.D == 128) && g.N % 16 == 0 && (long long)g.D * g.L * 2 <= 0x7FFFFFF0ll;
}

hipError_t launch_softmax_bwd_mfma(const Geometry& g, const uint16_t* q, const uint16_t* k,
                                   const uint16_t* v, const uint16_t* do_hm, const uint16_t* kt,
                                   const uint16_t* qt, const uint16_t* dot, const float* lse,
                                   const float* Dq, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                                   const SoftmaxBwdText& tx, float scale, hipStream_t s) {
  if (g.Ts > 0 && (!tx.k_text || !tx.v_text || !tx.ktt || !tx.dk_text || !tx.dv_text ||
                   tx.tpitch < (g.Ts + 15) / 16 * 16))
    return hipErrorInvalidValue;
  BwdArgs a;
  a.g = g;
  a.q = q; a.k = k; a.v = v; a.dO = do_hm; a.kt = kt; a.qt = qt; a.dOt = dot;
  a.lse = lse; a.Dq = Dq; a.dq = dq; a.dk = dk; a.dv = dv;
  a.k_text = (const bf16_t*)tx.k_text; a.v_text = (const bf16_t*)tx.v_text; a.ktt = tx.ktt;
  a.dk_text = (bf16_t*)tx.dk_text; a.dv_text = (bf16_t*)tx.dv_text; a.tpitch = tx.tpitch;
  a.ntext = 0;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  BwdArgs b = a;
  a.w = window_work(g, kBwdQW * 32);
  b.w = window_work(g, kBwdFW * 16);
  b.ntext = text_items_padded(g, kBwdFW * 16);
  if (a.w.grid == 0) return hipSuccess;
  const unsigned gk = (unsigned)(b.ntext + b.w.grid);
  const bool tq = g.Ts > 0;
  if (g.D == 128) {
    if (tq) softmax_bwd_dq_mfma_kernel<128, true><<<a.w.grid, kBwdQW * 64, 0, s>>>(a);
    else softmax_bwd_dq_mfma_kernel<128, false><<<a.w.grid, kBwdQW * 64, 0, s>>>(a);
    softmax_bwd_dkdv16_kernel<128><<<gk, kBwdFW * 64, 0, s>>>(b);
  } else {
    if (tq) softmax_bwd_dq_mfma_kernel<64, true><<<a.w.grid, kBwdQW * 64, 0, s>>>(a);
    else softmax_bwd_dq_mfma_kernel<64, false><<<a.w.grid, kBwdQW * 64, 0, s>>>(a);
    softmax_bwd_dkdv16_kernel<64><<<gk, kBwdFW * 64, 0, s>>>(b);
  }
  return hipGetLastError();
}

template hipError_t launch_softmax_bwd_prep<float>(const Geometry&, const float*, const float*,
                                                   const float*, float*, float*, float*, hipStream_t);
template hipError_t launch_softmax_bwd_prep<bf16_t>(const Geometry&, const bf16_t*, const bf16_t*,
                                                    const float*, bf16_t*, float*, float*,
                                                    hipStream_t);
template hipError_t launch_softmax_bwd_simt<float>(const Geometry&, const float*, const float*,
                                                   const float*, const float*, const float*,
                                                   const float*, float*, float*, float*,
                                                   const SoftmaxBwdText&, float, hipStream_t);
template hipError_t launch_softmax_bwd_simt<bf16_t>(const Geometry&, const bf16_t*, const bf16_t*,
                                                    const bf16_t*, const bf16_t*, const float*,
                                                    const float*, bf16_t*, bf16_t*, bf16_t*,
                                                    const SoftmaxBwdText&, float, hipStream_t);

}  // namespace vdn
