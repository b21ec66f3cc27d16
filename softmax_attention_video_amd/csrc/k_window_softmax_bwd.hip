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

#include <type_traits>

namespace vdn {

// ---------------------------------------------------------------------------
// Preprocess: dO (head-major) = g * dOhat, Dq = g * rowsum(dOhat * O),
// dg = rowsum(dOhat * O).  dOhat and O in the output layout [B,L,H,D].
// One thread per 8 channels of a (b, l, h) row; a row's D/8 lanes reduce
// with shuffles.  VEC: bf16 rows read as one 16-byte access per tensor
// (both pointers 16-byte aligned) instead of eight 2-byte loads.
// ---------------------------------------------------------------------------
template <typename T, bool VEC>
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
  if constexpr (VEC) {
    u32x4 xv = {0, 0, 0, 0}, yv = {0, 0, 0, 0};
    if (live) {
      xv = ld16(dout + src);
      yv = ld16(o + src);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(xv[i] << 16);
      x[2 * i + 1] = __uint_as_float(xv[i] & 0xFFFF0000u);
      y[2 * i] = __uint_as_float(yv[i] << 16);
      y[2 * i + 1] = __uint_as_float(yv[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      x[j] = live ? Elem<T>::load(dout, src + j) : 0.f;
      y[j] = live ? Elem<T>::load(o, src + j) : 0.f;
    }
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
  const unsigned grid = (unsigned)((n + 255) / 256);
  if constexpr (std::is_same<T, bf16_t>::value) {
    if ((((uintptr_t)o | (uintptr_t)dout) & 15) == 0) {
      softmax_bwd_prep_kernel<T, true><<<grid, 256, 0, s>>>(g, o, dout, g_s, do_hm, Dq, dg);
      return hipGetLastError();
    }
  }
  softmax_bwd_prep_kernel<T, false><<<grid, 256, 0, s>>>(g, o, dout, g_s, do_hm, Dq, dg);
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
// bf16 MFMA kernels (D = 64, 128; N % 16 == 0) with fp32 accumulation on
// v_mfma_f32_32x32x16_bf16.
// Tiles are staged global -> registers -> LDS (dQ: requested two tiles
// ahead; dK, dV: one) with one workgroup barrier per tile; rows past a
// span's end read as zero through the buffer descriptors.
//
// dQ (query-stationary, 8 waves x 32 queries): per 32-key block
//   S^T  = K Q^T        (A: K rows from LDS, B: the wave's Q fragments)
//   dP^T = V dO^T       (A: V rows from LDS, B: the wave's dO fragments)
//   dS^T = P^T (dP^T - Dq),  P^T = exp2(S^T scale log2e - lse log2e)
//   dQ^T += K^T dS^T    (A: K^T by transposing reads of the K rows, B: dS^T
//                        from registers)
// lse and Dq are per lane (one query per lane).
// ---------------------------------------------------------------------------
struct BwdArgs {
  Geometry g;
  SoftmaxWork w;
  const bf16_t* q;      // [B,H,L,D]
  const bf16_t* k;
  const bf16_t* v;
  const bf16_t* dO;     // g_s * dOhat, [B,H,L,D]
  const float* lse;     // [B,H,L], natural log
  const float* Dq;      // [B,H,L]
  bf16_t* dq;
  bf16_t* dk;
  bf16_t* dv;
  // text keys (g.Ts > 0): k_text, v_text [B,H,Ts,D] and the gradients
  // dk_text, dv_text [B,H,Ts,D]
  const bf16_t* k_text;
  const bf16_t* v_text;
  bf16_t* dk_text;
  bf16_t* dv_text;
  int ntext;            // leading workgroups of the dK/dV kernel that take text keys
  float scale, scale_log2;
};



constexpr int kBwdQW = 8;          // dQ kernel: waves (32 queries each)
constexpr int kBwdBK = 64;         // keys per staged tile (dQ) / queries per staged tile (dK, dV)

template <int D, bool TEXT>
__global__ __launch_bounds__(kBwdQW * 64) void softmax_bwd_dq_mfma_kernel(BwdArgs a) {
  constexpr int NT = kBwdQW * 64, BQ = kBwdQW * 32, BK = kBwdBK;
  // tile row r starts at r (2 D + 64) + 16 (r / 8) bytes, which keeps the
  // 16-byte row reads of 32 rows and the transposing reads of 8 consecutive
  // rows x 64 bytes free of bank conflicts (as in the dK / dV kernel)
  constexpr int KP = D + 32;
  constexpr int TS = BK * KP + BK;   // tile size (elements)
  auto rbase = [](int r) { return r * KP + (r >> 3) * 8; };
  // operand read-ahead of the products, in steps (the text variant holds
  // more registers and takes one)
  constexpr int AH = TEXT ? 1 : 2;
  constexpr int NKK = D / 16, NDB = D / 32, NB = BK / 32;
  constexpr int RCH = BK * D / 8 / NT;   // 16-byte chunks per thread
  static_assert(RCH * NT * 8 == BK * D, "tile split");
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][TS];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][TS];
  const Geometry& g = a.g;
  Item it;
  int q0;
  if (!decode_item<TEXT>(g, a.w, BQ, blockIdx.x, TEXT ? g.Ts : 0, it, q0)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hg = lane >> 5, l32 = lane & 31;
  const long long L = g.L;
  const size_t hb = (size_t)it.bh * L * D;
  const bf16_t* K = a.k + hb;
  const bf16_t* V = a.v + hb;
  // text keys (walk positions from L on)
  const size_t hbt = TEXT ? (size_t)it.bh * g.Ts * D : 0;
  const bf16_t* KT = TEXT ? a.k_text + hbt : nullptr;
  const bf16_t* VT = TEXT ? a.v_text + hbt : nullptr;
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
  u32x4 cA[2 * RCH], cB[2 * RCH];   // staging registers of even / odd tiles
  auto load_tile = [&](u32x4* cr, int j) {
    int ks, nk;
    walk.tile(j, ks, nk);
    const bool tx = TEXT && ks >= L;
    const int kr = tx ? ks - (int)L : ks;                // row in its own key array
    const rsrc_t rk = make_rsrc((tx ? KT : K) + (size_t)kr * D, (uint32_t)nk * D * 2);
    const rsrc_t rv = make_rsrc((tx ? VT : V) + (size_t)kr * D, (uint32_t)nk * D * 2);
#pragma unroll
    for (int i = 0; i < RCH; ++i) {
      const int c = tid + NT * i;
      const uint32_t off = (uint32_t)((c / (D / 8)) * D + (c % (D / 8)) * 8) * 2;
      cr[i] = buf_ld16(rk, off);
      cr[RCH + i] = buf_ld16(rv, off);
    }
  };
  auto store_tile = [&](const u32x4* cr, int buf) {
#pragma unroll
    for (int i = 0; i < RCH; ++i) {
      const int c = tid + NT * i;
      const int off = rbase(c / (D / 8)) + (c % (D / 8)) * 8;
      st16(&Ks[buf][off], cr[i]);
      st16(&Vs[buf][off], cr[RCH + i]);
    }
  };
  // In S^T a lane holds one query (lane % 32) and the keys 8 a + 4 hg + b of
  // the block (register 4 a + b); registers 8 h2 .. 8 h2 + 7 are the slots of
  // k-step h2 of dQ^T += K^T dS^T, whose K^T operand comes from the K rows
  // through the transposing read: lane group g takes rows d = 32 b + 16 (g %
  // 2) + 0..15 and the keys 16 h2 + 8 e + 4 (g / 2) + 0..3 of the block (e =
  // 0, 1: the two reads)
  const int grp = lane >> 4, sl = lane & 15;
  const int kt_off = (4 * (grp >> 1) + (sl >> 2)) * KP + 16 * (grp & 1) + 4 * (sl & 3);
  // tiles are requested two ahead of their LDS store: tile j + 2 into the
  // register set of its parity at the start of tile j, tile j + 1 (requested
  // a tile earlier) stored at its end
  if (walk.n > 0) {
    load_tile(cA, 0);
    store_tile(cA, 0);
  }
  if (walk.n > 1) load_tile(cB, 1);
  __syncthreads();
  auto tile_body = [&](int j, u32x4* c_next, u32x4* c_far) {
    const int buf = j & 1;
    int ks, nk;
    walk.tile(j, ks, nk);
    if (j + 2 < walk.n) load_tile(c_far, j + 2);
    const bf16_t* Kb = Ks[buf];
    const bf16_t* Vb = Vs[buf];
#pragma unroll
    for (int blk = 0; blk < NB; ++blk) {
      // S^T and dP^T; the K and V fragments of k-step kk + AH are read while
      // the products of k-step kk run
      f32x16 s = {}, dp = {};
      const bf16_t* kr = Kb + rbase(blk * 32 + l32) + hg * 8;
      const bf16_t* vr = Vb + rbase(blk * 32 + l32) + hg * 8;
      u32x4 fk[NKK], fv[NKK];
#pragma unroll
      for (int kk = 0; kk < AH; ++kk) {
        fk[kk] = ld16(kr + kk * 16);
        fv[kk] = ld16(vr + kk * 16);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * AH, 0);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk + AH < NKK) {
          fk[kk + AH] = ld16(kr + (kk + AH) * 16);
          fv[kk + AH] = ld16(vr + (kk + AH) * 16);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        s = mfma32x32x16(as_bf16x8(fk[kk]), qf[kk], s);
        dp = mfma32x32x16(as_bf16x8(fv[kk]), df[kk], dp);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // keys past the tile's valid ones (a partial last block) get P = 0
      const int nvb = nk - blk * 32;
      bf16x8 pb[2];
      if (nvb >= 32) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = fast_exp2(fmaf(s[i], a.scale_log2, -lse2));
          pb[i >> 3][i & 7] = static_cast<__bf16>(p * (dp[i] - dqv));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool vk = 8 * (i >> 2) + 4 * hg + (i & 3) < nvb;
          const float p = vk ? fast_exp2(fmaf(s[i], a.scale_log2, -lse2)) : 0.f;
          pb[i >> 3][i & 7] = static_cast<__bf16>(p * (dp[i] - dqv));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // dQ^T += K^T dS^T, step i = h2 NDB + b; the operands of step i + AH
      // are read while step i runs
      constexpr int NS = 2 * NDB;
      u32x2 ft[NS][2];
      auto kt_frags = [&](int i) {
        const int h2 = i / NDB, b = i % NDB;
        ft[i][0] = lds_read_tr16(Kb + rbase(blk * 32 + 16 * h2) + b * 32 + kt_off);
        ft[i][1] = lds_read_tr16(Kb + rbase(blk * 32 + 16 * h2 + 8) + b * 32 + kt_off);
      };
#pragma unroll
      for (int i = 0; i < AH; ++i) kt_frags(i);
      __builtin_amdgcn_sched_group_barrier(0x100, 2 * AH, 0);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (i + AH < NS) {
          kt_frags(i + AH);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        const int h2 = i / NDB, b = i % NDB;
        acc[b] = mfma32x32x16(as_bf16x8(u32x4{ft[i][0][0], ft[i][0][1], ft[i][1][0], ft[i][1][1]}),
                              pb[h2], acc[b]);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (j + 1 < walk.n) store_tile(c_next, buf ^ 1);
    __syncthreads();
  };
  for (int j = 0; j < walk.n; j += 2) {
    tile_body(j, cB, cA);
    if (j + 1 < walk.n) tile_body(j + 1, cA, cB);
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

// dK and dV together, one wave per 32 keys on 32 x 32 x 16 products (8
// waves, 256 keys per workgroup, two waves per SIMD): each operand fragment
// read from LDS then feeds a 32 x 32 block, half the LDS reads per flop of
// 16-key waves.  Per 32-query block of a staged 64-query tile:
//   S  = Q K^T,  dP = dO V^T      (A: Q / dO rows from LDS; B: the wave's K
//                                  fragments in registers / its V rows in LDS)
//   P = exp2(S scale log2e - lse log2e),  dS = P (dP - Dq)
//   dV^T += dO^T P,  dK^T += Q^T dS   (A: dO^T / Q^T from the row tiles by
//                                      transposing reads; B: P / dS)
// In S a lane holds one key (lane % 32) and the queries 8 a + 4 h + b of the
// block (register 4 a + b, h = lane / 32).  Registers 8 s .. 8 s + 7 are the
// eight contraction slots of k-step s of the accumulations; the matching A
// operand is two transposing reads of four queries each, 16 s + 4 h + 0..3
// and 16 s + 8 + 4 h + 0..3.
// LDS banks: a transposing 8-byte read is served for all 64 lanes at once,
// here 8 consecutive rows x 64 bytes, and a 16-byte row read per half-wave
// (32 rows, one 16-byte chunk each).  Row r of the Q and dO tiles starts at
// r (2 D + 64) + 16 (r / 8) bytes: 8 consecutive rows start in 8 different
// 64-byte bank groups, and the 4 rows of a 32-row block that share one are
// 16 bytes apart, so both reads are free of bank conflicts.  The wave's V
// rows see only row reads (pitch 304 / 144 bytes).
constexpr int kBwdKW = 8;          // 32-key dK / dV kernel: waves
// Operand read-ahead of the S / dP products and of the accumulations (in
// steps); deeper read-ahead spills at D = 128.
constexpr int kSdpAhead = 1;
constexpr int kAccAhead = 1;
template <int D>
__global__ __launch_bounds__(kBwdKW * 64) void softmax_bwd_dkdv_mfma_kernel(BwdArgs a) {
  constexpr int NT = kBwdKW * 64, BKEY = kBwdKW * 32, BQ = kBwdBK;
  constexpr int KP = D + 32;                 // Q / dO row tiles (elements), plus 8 per 8 rows
  constexpr int VP = D == 128 ? 152 : 72;    // the wave's V rows
  constexpr int NKK = D / 16, NDB = D / 32, NB = BQ / 32;
  constexpr int RCH = BQ * D / 8 / NT;
  constexpr int VCH = 32 * D / 8 / 64;   // 16-byte chunks per lane of the wave's V rows
  static_assert(RCH * NT * 8 == BQ * D && NB == 2, "tile split");
  constexpr int TS = BQ * KP + BQ;           // tile size (elements)
  auto rbase = [](int r) { return r * KP + (r >> 3) * 8; };   // start of tile row r
  __shared__ __attribute__((aligned(16))) bf16_t Qs[2][TS];
  __shared__ __attribute__((aligned(16))) bf16_t Ds[2][TS];
  __shared__ __attribute__((aligned(16))) bf16_t Vw[kBwdKW][32 * VP];
  __shared__ __attribute__((aligned(16))) float Ls[2][BQ];
  __shared__ __attribute__((aligned(16))) float Dd[2][BQ];
  const Geometry& g = a.g;
  Item it;
  int k0;
  bool text;
  if (!decode_key_item(g, a.w, BKEY, a.ntext, blockIdx.x, it, k0, text)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hg = lane >> 5, l32 = lane & 31;
  const int grp = lane >> 4, l16 = lane & 15;
  const long long L = g.L;
  const size_t hb = (size_t)it.bh * L * D;
  const size_t hk = text ? (size_t)it.bh * g.Ts * D : hb;
  const bf16_t* Kk = text ? a.k_text : a.k;
  const bf16_t* Vk = text ? a.v_text : a.v;
  bf16_t* dKk = text ? a.dk_text : a.dk;
  bf16_t* dVk = text ? a.dv_text : a.dv;
  const bf16_t* Q = a.q + hb;
  const bf16_t* dO = a.dO + hb;
  const float* lse = a.lse + (size_t)it.bh * L;
  const float* Dq = a.Dq + (size_t)it.bh * L;
  const int kw0 = k0 + wave * 32;   // the wave's first key
  const int krow = kw0 + l32;
  const bool kvalid = krow < it.q_end;
  bf16x8 kf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    u32x4 x = {0, 0, 0, 0};
    if (kvalid) x = ld16(Kk + hk + (size_t)krow * D + kk * 16 + hg * 8);
    kf[kk] = as_bf16x8(x);
  }
  bf16_t* Vme = Vw[wave];
#pragma unroll
  for (int i = 0; i < VCH; ++i) {
    const int c = lane + 64 * i, r = c / (D / 8), c8 = c % (D / 8);
    u32x4 x = {0, 0, 0, 0};
    if (kw0 + r < it.q_end) x = ld16(Vk + hk + (size_t)(kw0 + r) * D + c8 * 8);
    st16(Vme + r * VP + c8 * 8, x);
  }
  f32x16 accK[NDB], accV[NDB];
#pragma unroll
  for (int t = 0; t < NDB; ++t) {
    accK[t] = f32x16{};
    accV[t] = f32x16{};
  }
  const SpanWalk<BQ, 3> walk(it);
  u32x4 c0r[2 * RCH];
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
      const int off = rbase(c / (D / 8)) + (c % (D / 8)) * 8;
      st16(&Qs[buf][off], c0r[i]);
      st16(&Ds[buf][off], c0r[RCH + i]);
    }
  };
  auto load_piece1 = [&](int j) {      // lse and Dq
    int qs, nq;
    walk.tile(j, qs, nq);
    if (tid < BQ) {
      cl = tid < nq ? lse[qs + tid] * kLog2e : INFINITY;
      cd = tid < nq ? Dq[qs + tid] : 0.f;
    }
  };
  auto store_piece1 = [&](int buf) {
    if (tid < BQ) {
      Ls[buf][tid] = cl;
      Dd[buf][tid] = cd;
    }
  };
  // S and dP of query block qb.  The fragments of k-step kk + kSdpAhead are
  // read while the products of k-step kk run.
  auto sdp = [&](int buf, int qb, f32x16& sv, f32x16& dpv) {
    sv = f32x16{};
    dpv = f32x16{};
    const bf16_t* qr = &Qs[buf][rbase(qb * 32 + l32) + hg * 8];
    const bf16_t* dr = &Ds[buf][rbase(qb * 32 + l32) + hg * 8];
    const bf16_t* vr = Vme + l32 * VP + hg * 8;
    auto roff = [](int kk) { return kk * 16; };
    u32x4 fq[NKK], fd[NKK], fv[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (kk == 0) {
#pragma unroll
        for (int u = 0; u < kSdpAhead; ++u) {
          fq[u] = ld16(qr + roff(u));
          fd[u] = ld16(dr + roff(u));
          fv[u] = ld16(vr + u * 16);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 3 * kSdpAhead, 0);
      }
      if (kk + kSdpAhead < NKK) {
        fq[kk + kSdpAhead] = ld16(qr + roff(kk + kSdpAhead));
        fd[kk + kSdpAhead] = ld16(dr + roff(kk + kSdpAhead));
        fv[kk + kSdpAhead] = ld16(vr + (kk + kSdpAhead) * 16);
      }
      sv = mfma32x32x16(as_bf16x8(fq[kk]), kf[kk], sv);
      dpv = mfma32x32x16(as_bf16x8(fd[kk]), as_bf16x8(fv[kk]), dpv);
      if (kk + kSdpAhead < NKK) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    }
  };
  // P and dS as bf16 operands: register r of S is query 8 (r / 4) + 4 hg + r % 4
  auto probs = [&](int buf, int qb, const f32x16& sv, const f32x16& dpv, bf16x8* pb, bf16x8* db) {
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int q = qb * 32 + 8 * a4 + 4 * hg;
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(&Ls[buf][q]);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(&Dd[buf][q]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * a4 + e;
        const float pv = fast_exp2(fmaf(sv[r], a.scale_log2, -l4[e]));
        pb[r >> 3][r & 7] = static_cast<__bf16>(pv);
        db[r >> 3][r & 7] = static_cast<__bf16>(pv * (dpv[r] - d4[e]));
      }
    }
  };
  // transposing reads: group lane l16 points at query row 16 s + 8 e + 4 (grp
  // / 2) + l16 / 4 of the block (e = 0, 1: the two reads), channels 32 t + 16
  // (grp % 2) + 4 (l16 % 4) .. + 3
  const int tr_off = (4 * (grp >> 1) + (l16 >> 2)) * KP + 16 * (grp & 1) + 4 * (l16 & 3);
  constexpr int NACC = 2 * NDB;   // accumulation steps (k-step st, row block t) per query block
  // operands of accumulation step i = st NDB + t: dO^T and Q^T, two reads each
  auto acc_frags = [&](int buf, int qb, int i, u32x2* f) {
    const int st = i / NDB, t = i % NDB;
    const int o0 = rbase(qb * 32 + 16 * st) + 32 * t + tr_off;
    const int o1 = rbase(qb * 32 + 16 * st + 8) + 32 * t + tr_off;
    f[0] = lds_read_tr16(&Ds[buf][o0]);
    f[1] = lds_read_tr16(&Ds[buf][o1]);
    f[2] = lds_read_tr16(&Qs[buf][o0]);
    f[3] = lds_read_tr16(&Qs[buf][o1]);
  };
  // The operands of step i + kAccAhead are read while step i runs.
  auto accum = [&](int buf, int qb, const bf16x8* pb, const bf16x8* db) {
    u32x2 f[NACC][4];
#pragma unroll
    for (int i = 0; i < kAccAhead; ++i) acc_frags(buf, qb, i, f[i]);
#pragma unroll
    for (int i = 0; i < NACC; ++i) {
      if (i + kAccAhead < NACC) acc_frags(buf, qb, i + kAccAhead, f[i + kAccAhead]);
      const int st = i / NDB, t = i % NDB;
      accV[t] = mfma32x32x16(as_bf16x8(u32x4{f[i][0][0], f[i][0][1], f[i][1][0], f[i][1][1]}), pb[st], accV[t]);
      accK[t] = mfma32x32x16(as_bf16x8(u32x4{f[i][2][0], f[i][2][1], f[i][3][0], f[i][3][1]}), db[st], accK[t]);
      if (i + kAccAhead < NACC) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
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
    const int jn = j + 1 < walk.n ? j + 1 : j;
    load_piece0(jn);
    load_piece1(jn);
#pragma unroll
    for (int qb = 0; qb < NB; ++qb) {
      f32x16 sv, dpv;
      bf16x8 pb[2], db[2];
      sdp(buf, qb, sv, dpv);
      __builtin_amdgcn_sched_barrier(0);
      probs(buf, qb, sv, dpv, pb, db);
      __builtin_amdgcn_sched_barrier(0);
      accum(buf, qb, pb, db);
      __builtin_amdgcn_sched_barrier(0);
    }
    store_piece0(buf ^ 1);
    store_piece1(buf ^ 1);
    __syncthreads();
  }
  if (!kvalid) return;
  bf16_t* krk = dKk + hk + (size_t)krow * D;
  bf16_t* krv = dVk + hk + (size_t)krow * D;
#pragma unroll
  for (int t = 0; t < NDB; ++t)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int d = 32 * t + 8 * a4 + 4 * hg;
      u32x2 pk, pv;
      pk[0] = pack_bf16x2(accK[t][4 * a4 + 0] * a.scale, accK[t][4 * a4 + 1] * a.scale);
      pk[1] = pack_bf16x2(accK[t][4 * a4 + 2] * a.scale, accK[t][4 * a4 + 3] * a.scale);
      pv[0] = pack_bf16x2(accV[t][4 * a4 + 0], accV[t][4 * a4 + 1]);
      pv[1] = pack_bf16x2(accV[t][4 * a4 + 2], accV[t][4 * a4 + 3]);
      *reinterpret_cast<u32x2*>(krk + d) = pk;
      *reinterpret_cast<u32x2*>(krv + d) = pv;
    }
}

bool softmax_bwd_mfma_ok(const Geometry& g) {
  return (g.D == 64 || g.D == 128) && g.N % 16 == 0 && (long long)g.D * g.L * 2 <= 0x7FFFFFF0ll;
}

hipError_t launch_softmax_bwd_mfma(const Geometry& g, const uint16_t* q, const uint16_t* k,
                                   const uint16_t* v, const uint16_t* do_hm, const float* lse,
                                   const float* Dq, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                                   const SoftmaxBwdText& tx, float scale, hipStream_t s) {
  if (g.Ts > 0 && (!tx.k_text || !tx.v_text || !tx.dk_text || !tx.dv_text))
    return hipErrorInvalidValue;
  BwdArgs a;
  a.g = g;
  a.q = q; a.k = k; a.v = v; a.dO = do_hm;
  a.lse = lse; a.Dq = Dq; a.dq = dq; a.dk = dk; a.dv = dv;
  a.k_text = (const bf16_t*)tx.k_text; a.v_text = (const bf16_t*)tx.v_text;
  a.dk_text = (bf16_t*)tx.dk_text; a.dv_text = (bf16_t*)tx.dv_text;
  a.ntext = 0;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  BwdArgs b = a;
  a.w = window_work(g, kBwdQW * 32);
  b.w = window_work(g, kBwdKW * 32);
  b.ntext = text_items_padded(g, kBwdKW * 32);
  if (a.w.grid == 0) return hipSuccess;
  const unsigned gk = (unsigned)(b.ntext + b.w.grid);
  const bool tq = g.Ts > 0;
  if (g.D == 128) {
    if (tq) softmax_bwd_dq_mfma_kernel<128, true><<<a.w.grid, kBwdQW * 64, 0, s>>>(a);
    else softmax_bwd_dq_mfma_kernel<128, false><<<a.w.grid, kBwdQW * 64, 0, s>>>(a);
    softmax_bwd_dkdv_mfma_kernel<128><<<gk, kBwdKW * 64, 0, s>>>(b);
  } else {
    if (tq) softmax_bwd_dq_mfma_kernel<64, true><<<a.w.grid, kBwdQW * 64, 0, s>>>(a);
    else softmax_bwd_dq_mfma_kernel<64, false><<<a.w.grid, kBwdQW * 64, 0, s>>>(a);
    softmax_bwd_dkdv_mfma_kernel<64><<<gk, kBwdKW * 64, 0, s>>>(b);
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
