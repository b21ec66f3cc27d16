// VDA readout and linear-branch epilogue.
//
// Paper ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream
// Video Generation"), method, bidirectional linear attention: at readout
// time the state just outside the query frame's window is gathered from each
// directional scan, the accumulated channel-wise decay across the skipped
// local span is applied, the query is evaluated against the resulting
// memory and the two readouts are added.  Branch calibration: the linear
// readout is RMS-normalised and passed through its own output gate.
// System section (VDA-Gather, VDA-Epilogue): gather + decay bridge, then
// RMSNorm + gating + layout conversion, here fused into one kernel.
//
// For query frame t in chunk c (non-anchor):
//   i_fwd = max(c - wc, 0), ws = i_fwd * cf, i_rev = min(c + wc + 1, C),
//   we = min(i_rev * cf, F) - 1;  anchor frames: 0, 0, C, F - 1.
//   M_t = diag(prod_{f=ws..t} alpha_f) P_fwd[i_fwd] + diag(prod_{f=t..we} alpha_f) P_rev[i_rev]
//   O_l = q M_t;  out = g_l * gamma * O_l / sqrt(mean(O_l^2) + eps)   in [B, L, H, D]
#include "vdn_common.h"
#include "vdn_internal.h"

namespace vdn {

template <typename T, int D>
__global__ __launch_bounds__(256) void vda_readout_simt_kernel(Geometry g, const T* __restrict__ q,
                                                               const float* __restrict__ alpha,
                                                               const float* __restrict__ P_fwd,
                                                               const float* __restrict__ P_rev,
                                                               const float* __restrict__ g_l,
                                                               const float* __restrict__ gamma,
                                                               float eps, T* __restrict__ out) {
  constexpr int TPG = 16;          // threads per token
  constexpr int CPT = D / TPG;     // output columns per thread
  constexpr int TOK = 256 / TPG;   // tokens per pass
  __shared__ __attribute__((aligned(16))) float Ms[D * D];
  __shared__ float Qs[TOK][D + 1];
  __shared__ float dfs[D], drs[D];

  const int t = blockIdx.x % g.F;
  const int bh = blockIdx.x / g.F;
  const int tid = threadIdx.x;
  int i_f, ws, i_r, we;
  readout_indices(g, t, i_f, ws, i_r, we);
  const float* al = alpha + (size_t)bh * g.F * D;
  for (int k = tid; k < D; k += 256) {
    float df = 1.f, dr = 1.f;
    for (int f = ws; f <= t; ++f) df *= al[(size_t)f * D + k];
    for (int f = t; f <= we; ++f) dr *= al[(size_t)f * D + k];
    dfs[k] = df;
    drs[k] = dr;
  }
  __syncthreads();
  const size_t DD = (size_t)D * D;
  const float* pf = P_fwd + ((size_t)bh * (g.C + 1) + i_f) * DD;
  const float* pr = P_rev + ((size_t)bh * (g.C + 1) + i_r) * DD;
  for (int e = tid; e < D * D; e += 256) {
    const int k = e / D;
    Ms[e] = dfs[k] * pf[e] + drs[k] * pr[e];
  }

  const int grp = tid / TPG, sub = tid % TPG;
  float gm[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) gm[j] = gamma ? gamma[sub * CPT + j] : 1.f;
  const int bidx = bh / g.H, h = bh % g.H;
  const size_t tok0 = (size_t)bh * g.L + (size_t)t * g.N;   // row of token 0 of frame t
  for (int n0 = 0; n0 < g.N; n0 += TOK) {
    __syncthreads();
    for (int e = tid; e < TOK * D; e += 256) {
      const int r = e / D, c = e % D;
      Qs[r][c] = (n0 + r < g.N) ? Elem<T>::load(q, (tok0 + n0 + r) * D + c) : 0.f;
    }
    __syncthreads();
    float o[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) o[j] = 0.f;
    for (int k = 0; k < D; ++k) {
      const float qk = Qs[grp][k];
#pragma unroll
      for (int j = 0; j < CPT; ++j) o[j] = fmaf(qk, Ms[k * D + sub * CPT + j], o[j]);
    }
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) ss = fmaf(o[j], o[j], ss);
#pragma unroll
    for (int m = TPG / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, TPG);
    const int n = n0 + grp;
    if (n < g.N) {
      const float r = rsqrtf(ss / (float)D + eps);
      const size_t l = (size_t)t * g.N + n;
      const float gate = g_l[(size_t)bh * g.L + l] * r;
      const size_t ob = (((size_t)bidx * g.L + l) * g.H + h) * D + sub * CPT;
#pragma unroll
      for (int j = 0; j < CPT; ++j) Elem<T>::store(out, ob + j, o[j] * gate * gm[j]);
    }
  }
}

// bf16 path (D = 64, 128): one workgroup of 8 waves per (b, h, query
// frame).  M_t is built once in fp32, stored transposed in LDS as bf16 hi +
// lo parts, and O_l^T = M^T Q^T runs on v_mfma_f32_32x32x16_bf16 (hi and lo
// products accumulate in fp32, so M keeps ~16 extra mantissa bits: the
// entries of M cancel in q M, and a single bf16 rounding of M is visible in
// the output).  A lane ends up holding one token and half of its dv values:
// the RMS is an in-lane sum of squares plus one exchange with lane ^ 32.
// The normalised rows go through a per-wave LDS tile so that the stores
// write whole d_v-rows of [B, L, H, d_v] (16 bytes per lane, consecutive
// lanes along d_v): written straight from the MFMA layout, each store
// instruction would touch 32 rows H * d_v * 2 bytes apart with 8 bytes each.
constexpr int kReadoutNW = 8;   // waves per workgroup of the MFMA readout
template <int D>
__global__ __launch_bounds__(kReadoutNW * 64) void vda_readout_mfma_kernel(Geometry g, const bf16_t* __restrict__ q,
                                                               const float* __restrict__ alpha,
                                                               const float* __restrict__ P_fwd,
                                                               const float* __restrict__ P_rev,
                                                               const float* __restrict__ g_l,
                                                               const float* __restrict__ gamma,
                                                               float eps, bf16_t* __restrict__ out) {
  constexpr int MP = D + 8;        // pitch of M^T (bf16)
  constexpr int NKK = D / 16, NDB = D / 32;
  constexpr int OP = D + 8;        // pitch of the output tile (bf16)
  constexpr int RPI = 64 / (D / 8);   // token rows per 16-byte-per-lane pass
  constexpr int NT = kReadoutNW * 64, TSTEP = kReadoutNW * 32;
  __shared__ __attribute__((aligned(16))) bf16_t mh[D * MP];
  __shared__ __attribute__((aligned(16))) bf16_t ml[D * MP];
  __shared__ __attribute__((aligned(16))) bf16_t ot[kReadoutNW][32 * OP];
  __shared__ float dfs[D], drs[D];
  __shared__ __attribute__((aligned(16))) float gms[D];

  const int t = blockIdx.x % g.F;
  const int bh = blockIdx.x / g.F;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hg = lane >> 5, l32 = lane & 31;
  int i_f, ws, i_r, we;
  readout_indices(g, t, i_f, ws, i_r, we);
  const float* al = alpha + (size_t)bh * g.F * D;
  // decay bridges: thread (part, k) forms one channel's product over its
  // span, loading 4 frames at a time so the loads are in flight together
  if (tid < 2 * D) {
    const int k = tid % D, part = tid / D;
    const int f0 = part == 0 ? ws : t, f1 = part == 0 ? t : we;   // inclusive
    float d = 1.f;
    int f = f0;
    for (; f + 3 <= f1; f += 4) {
      const float a0 = al[(size_t)f * D + k], a1 = al[(size_t)(f + 1) * D + k];
      const float a2 = al[(size_t)(f + 2) * D + k], a3 = al[(size_t)(f + 3) * D + k];
      d *= a0;
      d *= a1;
      d *= a2;
      d *= a3;
    }
    for (; f <= f1; ++f) d *= al[(size_t)f * D + k];
    (part == 0 ? dfs : drs)[k] = d;
  }
  for (int k = tid; k < D; k += NT) gms[k] = gamma ? gamma[k] : 1.f;
  __syncthreads();
  const size_t DD = (size_t)D * D;
  const float* pf = P_fwd + ((size_t)bh * (g.C + 1) + i_f) * DD;
  const float* pr = P_rev + ((size_t)bh * (g.C + 1) + i_r) * DD;
  // M^T as bf16 hi + lo: each thread forms a pair of rows k, k + 1 of M for
  // four columns and stores them as packed 32-bit pairs of M^T
  for (int e = tid; e < (D / 2) * (D / 4); e += NT) {
    const int k = 2 * (e / (D / 4)), j0 = (e % (D / 4)) * 4;
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(pf + (size_t)k * D + j0);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(pf + (size_t)(k + 1) * D + j0);
    const f32x4 b0 = *reinterpret_cast<const f32x4*>(pr + (size_t)k * D + j0);
    const f32x4 b1 = *reinterpret_cast<const f32x4*>(pr + (size_t)(k + 1) * D + j0);
    const float f0 = dfs[k], f1 = dfs[k + 1], r0 = drs[k], r1 = drs[k + 1];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float m0 = f0 * a0[c] + r0 * b0[c];
      const float m1 = f1 * a1[c] + r1 * b1[c];
      const bf16_t h0 = f32_to_bf16(m0), h1 = f32_to_bf16(m1);
      const bf16_t l0 = f32_to_bf16(m0 - bf16_to_f32(h0)), l1 = f32_to_bf16(m1 - bf16_to_f32(h1));
      *reinterpret_cast<uint32_t*>(&mh[(j0 + c) * MP + k]) = (uint32_t)h0 | ((uint32_t)h1 << 16);
      *reinterpret_cast<uint32_t*>(&ml[(j0 + c) * MP + k]) = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
  }
  __syncthreads();

  const int bidx = bh / g.H, h = bh % g.H;
  const size_t tok0 = (size_t)bh * g.L + (size_t)t * g.N;
  // q fragments of the wave's next 32 tokens are requested while the
  // current ones are multiplied.  Buffer loads over the frame's rows: tokens
  // past the frame read as zeros, with no branch, so the wait counts stay
  // exact (a load under a lane-dependent branch makes every wait after it a
  // wait for all loads).
  const rsrc_t qrs = make_rsrc(q + tok0 * D, (uint32_t)g.N * D * 2);
  const rsrc_t grs = make_rsrc(g_l + (size_t)bh * g.L + (size_t)t * g.N, (uint32_t)g.N * 4);
  // the frame's rows of this head in [B, L, H, d_v]: row r at r * H * d_v;
  // the descriptor ends after row N - 1, so stores of rows past it are dropped
  const int HD = g.H * D;
  const rsrc_t ors = make_rsrc(out + (((size_t)bidx * g.L + (size_t)t * g.N) * g.H + h) * D,
                               (uint32_t)(((g.N - 1) * HD + D) * 2));
  bf16x8 qf[NKK];
  auto load_q = [&](int n0, bf16x8* dst) {
    const uint32_t off = (uint32_t)((n0 + l32) * D + hg * 8) * 2;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) dst[kk] = as_bf16x8(buf_ld16(qrs, off + kk * 32));
  };
  // the gate of the lane's token travels with its q fragments: a load issued
  // and consumed in one step would wait for that step's prefetch as well
  auto load_gate = [&](int n) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(grs, (int)(n * 4), 0, 0));
  };
  // Steps alternate between two fragment sets, so the next step's loads are
  // never copied (a copy at the end of a step would make the step wait for
  // them); each step requests the step after next.
  bf16x8 qb[NKK];
  float gate_a = load_gate(wave * 32 + l32), gate_b = 0.f;
  load_q(wave * 32, qf);
  auto step = [&](int n0, const bf16x8* cur, bf16x8* nxt, float gate_c, float& gate_nx) {
    const int n = n0 + l32;
    // M^T is read from LDS in every step: kept in registers for the frame it
    // would take ~256 of them (one wave per SIMD), which this fence forbids
    __asm__ volatile("" ::: "memory");
    load_q(n0 + TSTEP, nxt);
    gate_nx = load_gate(n + TSTEP);
    f32x16 o[NDB];
#pragma unroll
    for (int b = 0; b < NDB; ++b) {
      o[b] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int off = (b * 32 + l32) * MP + kk * 16 + hg * 8;
        o[b] = mfma32x32x16(as_bf16x8(ld16(&mh[off])), cur[kk], o[b]);
        o[b] = mfma32x32x16(as_bf16x8(ld16(&ml[off])), cur[kk], o[b]);
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) ss = fmaf(o[b][i], o[b][i], ss);
    ss = half_sum(ss);
    // tokens past the frame carry zeros (gate 0) and are not stored
    const float sc = gate_c * rsqrtf(ss / (float)D + eps);
    bf16_t* tile = ot[wave];
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const f32x4 gm = *reinterpret_cast<const f32x4*>(&gms[b * 32 + 8 * i4 + 4 * hg]);
        u32x2 pk;
        pk[0] = pack_bf16x2(o[b][i4 * 4 + 0] * sc * gm[0], o[b][i4 * 4 + 1] * sc * gm[1]);
        pk[1] = pack_bf16x2(o[b][i4 * 4 + 2] * sc * gm[2], o[b][i4 * 4 + 3] * sc * gm[3]);
        *reinterpret_cast<u32x2*>(&tile[l32 * OP + b * 32 + 8 * i4 + 4 * hg]) = pk;
      }
    // the wave reads back whole token rows and stores 16 bytes per lane
    // along d_v (a wave-scope fence orders the tile's writes and reads)
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    u32x4 rows[32 / RPI];
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it)
      rows[it] = ld16(&tile[(it * RPI + lane / (D / 8)) * OP + (lane % (D / 8)) * 8]);
#pragma unroll
    for (int it = 0; it < 32 / RPI; ++it) {
      const int r = n0 + it * RPI + lane / (D / 8);
      __builtin_amdgcn_raw_buffer_store_b128(rows[it], ors, (int)((r * HD + (lane % (D / 8)) * 8) * 2), 0, 0);
    }
  };
  for (int n0 = wave * 32; n0 < g.N; n0 += 2 * TSTEP) {
    step(n0, qf, qb, gate_a, gate_b);
    if (n0 + TSTEP < g.N) step(n0 + TSTEP, qb, qf, gate_b, gate_a);
  }
}

template <typename T>
hipError_t launch_vda_readout(const Geometry& g, const T* q, const float* alpha, const float* P_fwd,
                              const float* P_rev, const float* g_l, const float* gamma, float eps,
                              T* out, hipStream_t s) {
  const unsigned grid = (unsigned)(g.B * g.H * g.F);
  switch (g.D) {
    case 16: vda_readout_simt_kernel<T, 16><<<grid, 256, 0, s>>>(g, q, alpha, P_fwd, P_rev, g_l, gamma, eps, out); break;
    case 32: vda_readout_simt_kernel<T, 32><<<grid, 256, 0, s>>>(g, q, alpha, P_fwd, P_rev, g_l, gamma, eps, out); break;
    case 64: vda_readout_simt_kernel<T, 64><<<grid, 256, 0, s>>>(g, q, alpha, P_fwd, P_rev, g_l, gamma, eps, out); break;
    case 128: vda_readout_simt_kernel<T, 128><<<grid, 256, 0, s>>>(g, q, alpha, P_fwd, P_rev, g_l, gamma, eps, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <>
hipError_t launch_vda_readout<bf16_t>(const Geometry& g, const bf16_t* q, const float* alpha,
                                      const float* P_fwd, const float* P_rev, const float* g_l,
                                      const float* gamma, float eps, bf16_t* out, hipStream_t s) {
  const unsigned grid = (unsigned)(g.B * g.H * g.F);
  // the MFMA kernel addresses one frame of all heads with 32-bit buffer offsets
  const bool fits = (long long)g.N * g.H * g.D * 2 <= 0x7FFFFFF0ll;
  switch (g.D) {
    case 16: vda_readout_simt_kernel<bf16_t, 16><<<grid, 256, 0, s>>>(g, q, alpha, P_fwd, P_rev, g_l, gamma, eps, out); break;
    case 32: vda_readout_simt_kernel<bf16_t, 32><<<grid, 256, 0, s>>>(g, q, alpha, P_fwd, P_rev, g_l, gamma, eps, out); break;
    case 64:
      if (fits) vda_readout_mfma_kernel<64><<<grid, kReadoutNW * 64, 0, s>>>(g, q, alpha, P_fwd, P_rev, g_l, gamma, eps, out);
      else vda_readout_simt_kernel<bf16_t, 64><<<grid, 256, 0, s>>>(g, q, alpha, P_fwd, P_rev, g_l, gamma, eps, out);
      break;
    case 128:
      if (fits) vda_readout_mfma_kernel<128><<<grid, kReadoutNW * 64, 0, s>>>(g, q, alpha, P_fwd, P_rev, g_l, gamma, eps, out);
      else vda_readout_simt_kernel<bf16_t, 128><<<grid, 256, 0, s>>>(g, q, alpha, P_fwd, P_rev, g_l, gamma, eps, out);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template hipError_t launch_vda_readout<float>(const Geometry&, const float*, const float*,
                                              const float*, const float*, const float*,
                                              const float*, float, float*, hipStream_t);

}  // namespace vdn
