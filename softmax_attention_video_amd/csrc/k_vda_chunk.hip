// VDA chunk composition and the bidirectional chunk prefix scans.
//
// Paper ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream
// Video Generation"), system section, chunk-wise scans: each frame is an
// affine map S -> T_f S + U_f, and attention only reads memory at VAE-chunk
// boundaries, so the maps of each chunk are composed into one (T_c, U_c) and
// the shorter chunk sequence is scanned in both directions; the prompt state
// enters as the leading virtual frame.  Method, bidirectional linear
// attention: each directional scan starts from text_init_scale * S_text.
//
//   forward : T_c = T_{e} ... T_{s},  U_c = T_e(...(T_{s+1} U_s + U_{s+1})...) + U_e
//   reverse : the same frames applied from e down to s
//   P_fwd[0] = a S_text,  P_fwd[c+1] = T_c P_fwd[c] + U_c
//   P_rev[C] = a S_text,  P_rev[c]   = T_c P_rev[c+1] + U_c
//
// Every map acts column by column on the state, so the work splits over
// 32-column blocks: the composition runs one workgroup per
// (b, h, direction, chunk, column block of [T_c | U_c]) and the scan one per
// (b, h, direction, column block of P).  The left factor (a D x D fp32
// matrix) is staged in LDS; the 32 state columns stay in LDS between steps.
#include "vdn_common.h"
#include "vdn_internal.h"

namespace vdn {

constexpr int kCB = 32;   // state columns per workgroup

// Y_out[:, 0:32] = Ts * Y_in[:, 0:32] (+ add[:, 0:32] if add != nullptr).
// Ts: [D][D+1] in LDS; Y_in/Y_out: [D][32] in LDS; add: row-major, pitch ldadd.
template <int D>
__device__ __forceinline__ void apply_left(const float* Ts, const float* Y_in, float* Y_out,
                                           const float* add, int ldadd, int ncols) {
  constexpr int RPT = (D + 31) / 32;
  const int tx = threadIdx.x & 7, ty = threadIdx.x >> 3;
  float acc[RPT][4];
#pragma unroll
  for (int r = 0; r < RPT; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
  for (int k = 0; k < D; ++k) {
    const f32x4 y = *reinterpret_cast<const f32x4*>(&Y_in[k * kCB + tx * 4]);
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int row = ty + 32 * r;
      const float t = row < D ? Ts[row * (D + 1) + k] : 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(t, y[c], acc[r][c]);
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
      if (add && col < ncols) v += add[(size_t)row * ldadd + col];
      Y_out[row * kCB + col] = v;
    }
  }
}

template <int D>
__device__ __forceinline__ void stage_matrix(float* Ts, const float* src) {
  for (int e = threadIdx.x; e < D * D; e += blockDim.x) Ts[(e / D) * (D + 1) + (e % D)] = src[e];
}

// ---- composition: grid = B*H * 2 * C * (2D/32) ----
template <int D>
__global__ __launch_bounds__(256) void vda_chunk_compose_kernel(Geometry g, const float* __restrict__ Tf,
                                                                const float* __restrict__ Uf,
                                                                float* __restrict__ Tc,
                                                                float* __restrict__ Uc, int dirs_mask) {
  __shared__ __attribute__((aligned(16))) float smem[D * (D + 1) + 2 * D * kCB];
  float* Ts = smem;                        // D x (D+1)
  float* Y1 = smem + D * (D + 1);          // D x 32 (16-byte aligned: D*(D+1) % 4 == 0)
  float* Y0 = Y1 + D * kCB;                // D x 32
  constexpr int NCBH = (D + kCB - 1) / kCB;   // column blocks per half of [T | U]
  constexpr int NCB = 2 * NCBH;
  int id = blockIdx.x;
  const int cb = id % NCB; id /= NCB;
  const int c = id % g.C; id /= g.C;
  const int dir = id % 2;
  const int bh = id / 2;
  if (!((dirs_mask >> dir) & 1)) return;
  const size_t DD = (size_t)D * D;
  // columns [lc0, lc0 + ncols) of T (cb < NCBH) or of U
  const bool upart = cb >= NCBH;
  const int lc0 = (cb % NCBH) * kCB;
  const int ncols = min(kCB, D - lc0);
  const int s = c * g.cf, e = s + g.cf - 1;
  const int first = dir == 0 ? s : e;
  const int step = dir == 0 ? 1 : -1;
  const float* fbase_T = Tf + (size_t)bh * g.F * DD;
  const float* fbase_U = Uf + (size_t)bh * g.F * DD;

  // Y0 = columns of the first frame's map
  {
    const float* src = (upart ? fbase_U : fbase_T) + (size_t)first * DD;
    for (int i = threadIdx.x; i < D * kCB; i += blockDim.x) {
      const int row = i / kCB, col = i % kCB;
      Y0[i] = col < ncols ? src[(size_t)row * D + lc0 + col] : 0.f;
    }
  }
  float* yin = Y0;
  float* yout = Y1;
  for (int n = 1; n < g.cf; ++n) {
    const int f = first + step * n;
    __syncthreads();
    stage_matrix<D>(Ts, fbase_T + (size_t)f * DD);
    __syncthreads();
    apply_left<D>(Ts, yin, yout, upart ? fbase_U + (size_t)f * DD + lc0 : nullptr, D, ncols);
    float* t = yin; yin = yout; yout = t;
  }
  __syncthreads();
  float* dst = (upart ? Uc : Tc) + (((size_t)bh * 2 + dir) * g.C + c) * DD;
  for (int i = threadIdx.x; i < D * kCB; i += blockDim.x) {
    const int row = i / kCB, col = i % kCB;
    if (col < ncols) dst[(size_t)row * D + lc0 + col] = yin[i];
  }
}

// ---------------------------------------------------------------------------
// fp32 MFMA chain kernel (D = 64, 128): Y <- L_s Y (+ A_s), s = 0..S-1, on a
// 32-column block of Y, with v_mfma_f32_32x32x2f32.  Wave w owns rows
// 32w..32w+31: its slice of each left factor L_s goes straight from global
// memory into registers (the next step's slice is fetched while the current
// product runs), so the left factors never pass through LDS.  Y is kept
// transposed in LDS (Yt[n][k]) so both MFMA operands are k-contiguous; the
// contracted index is permuted identically on both operands (lane half g
// takes k = k0 + 4g .. k0 + 4g + 3 of each 8-wide group).
//
// Mode compose: grid (b, h, dir, chunk, part in {T, U}, column block);
//   Y0 = first frame's T or U columns, L_s = T of the next frames, A_s = U
//   of the next frames for part U; the final Y is T_c / U_c.
// Mode scan: grid (b, h, dir, column block); Y0 = init_scale * S_text,
//   L_s = T_c, A_s = U_c in scan order; Y is written to P after every step.
// Mode frame scan: the same grid and Y0, but L_s = T_f, A_s = U_f of the
//   frames themselves in scan order (no composition), Y written to P at
//   every chunk boundary.
// A workgroup holds kChainG column blocks of one chain, 256 threads each:
// the chains are latency-bound (one dependent product per step), so sharing
// a compute unit interleaves their matrix-core work on each SIMD instead of
// holding one compute unit per column block for the same time (two per
// workgroup keep the register budget for the left factors' prefetch).
// ---------------------------------------------------------------------------
constexpr int kChainG = 2;
template <int D>
__global__ __launch_bounds__(256 * kChainG) void vda_chain_mfma_kernel(Geometry g, const float* __restrict__ Tf,
                                                             const float* __restrict__ Uf,
                                                             float* __restrict__ Tc, float* __restrict__ Uc,
                                                             const float* __restrict__ S_text,
                                                             float init_scale, float* __restrict__ P_fwd,
                                                             float* __restrict__ P_rev, int mode,
                                                             int dirs_mask) {
  constexpr int NB = D / 32;            // row blocks (waves doing MFMA work)
  constexpr int NCB = D / 32;           // 32-column blocks of Y
  constexpr int YP = D + 4;             // pitch of Yt (floats)
  constexpr int NK8 = D / 8;            // 8-wide k groups
  static_assert(NCB % kChainG == 0, "column blocks per workgroup");
  __shared__ __attribute__((aligned(16))) float Yts[kChainG][32 * YP];
  const size_t DD = (size_t)D * D;
  const int grp = threadIdx.x >> 8;     // 256-thread group: one column block
  float* Yt = Yts[grp];
  const int tid = threadIdx.x & 255, wave = tid >> 6, lane = tid & 63, hg = lane >> 5, l32 = lane & 31;
  int id = blockIdx.x;
  const int cb = (id % (NCB / kChainG)) * kChainG + grp;
  id /= NCB / kChainG;
  int part = 0, c = 0, dir, bh;
  if (mode == 0) {
    part = id % 2; id /= 2;
    c = id % g.C; id /= g.C;
  }
  dir = id % 2;
  bh = id / 2;
  if (!((dirs_mask >> dir) & 1)) return;
  const int col0 = cb * 32;
  int nsteps;
  const float *L0, *A0 = nullptr;
  ptrdiff_t lstride;       // elements between consecutive left factors (signed: reverse order)
  const float* ysrc;
  float yscale = 1.f;
  float* out_final = nullptr;
  float* Pb = nullptr;
  if (mode == 0) {
    const int s0 = c * g.cf, e0 = s0 + g.cf - 1;
    const int first = dir == 0 ? s0 : e0;
    const int step = dir == 0 ? 1 : -1;
    nsteps = g.cf - 1;
    lstride = (ptrdiff_t)step * (ptrdiff_t)DD;
    L0 = Tf + ((size_t)bh * g.F + first + step) * DD;
    if (part == 1) A0 = Uf + ((size_t)bh * g.F + first + step) * DD;
    ysrc = (part == 0 ? Tf : Uf) + ((size_t)bh * g.F + first) * DD;
    out_final = (part == 0 ? Tc : Uc) + (((size_t)bh * 2 + dir) * g.C + c) * DD;
  } else {
    float* P = dir == 0 ? P_fwd : P_rev;
    lstride = (dir == 0 ? 1 : -1) * (ptrdiff_t)DD;
    if (mode == 1) {
      nsteps = g.C;
      const int c0 = dir == 0 ? 0 : g.C - 1;
      L0 = Tc + (((size_t)bh * 2 + dir) * g.C + c0) * DD;
      A0 = Uc + (((size_t)bh * 2 + dir) * g.C + c0) * DD;
    } else {
      nsteps = g.F;
      const int f0 = dir == 0 ? 0 : g.F - 1;
      L0 = Tf + ((size_t)bh * g.F + f0) * DD;
      A0 = Uf + ((size_t)bh * g.F + f0) * DD;
    }
    ysrc = S_text + (size_t)bh * DD;
    yscale = init_scale;
    Pb = P + (size_t)bh * (g.C + 1) * DD;
  }
  // Y0 -> Yt (transposed), and the initial P slot in scan mode
  for (int e = tid; e < D * 32; e += 256) {
    const int k = e / 32, n = e % 32;
    const float y = yscale * ysrc[(size_t)k * D + col0 + n];
    Yt[n * YP + k] = y;
    if (Pb) Pb[(size_t)(dir == 0 ? 0 : g.C) * DD + (size_t)k * D + col0 + n] = y;
  }
  const bool mw = wave < NB;           // waves holding a row block
  const int mrow = wave * 32 + l32;    // this lane's row of the left factor
  f32x4 lf[NK8], lnext[NK8];
  auto load_left = [&](const float* Lm, f32x4 (&dst)[NK8]) {
#pragma unroll
    for (int j = 0; j < NK8; ++j)
      dst[j] = mw ? *reinterpret_cast<const f32x4*>(Lm + (size_t)mrow * D + 8 * j + 4 * hg) : f32x4{};
  };
  // the additive term's 32 x 32 block of this lane group, in accumulator
  // layout; fetched one step ahead like the left factor
  float af[16], anext[16];
  auto load_add = [&](const float* Am, float (&dst)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i)
      dst[i] = mw && Am ? Am[(size_t)(wave * 32 + mfma32_row(i, hg)) * D + col0 + l32] : 0.f;
  };
  if (nsteps > 0) {
    load_left(L0, lf);
    load_add(A0, af);
  }
  for (int st = 0; st < nsteps; ++st) {
    const float* Lm = L0 + st * lstride;
    if (st + 1 < nsteps) {
      load_left(Lm + lstride, lnext);
      load_add(A0 ? A0 + (st + 1) * lstride : nullptr, anext);
    }
    __syncthreads();                      // Yt holds the current Y
    f32x16 acc = f32x16{};
    if (mw) {
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = af[i];
#pragma unroll
      for (int j = 0; j < NK8; ++j) {
        const f32x4 yb = *reinterpret_cast<const f32x4*>(&Yt[l32 * YP + 8 * j + 4 * hg]);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc = mfma32x32x2f32(lf[j][q], yb[q], acc);
      }
    }
    __syncthreads();                      // everyone has read the old Y
    if (mw) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        f32x4 v = {acc[4 * i4], acc[4 * i4 + 1], acc[4 * i4 + 2], acc[4 * i4 + 3]};
        *reinterpret_cast<f32x4*>(&Yt[l32 * YP + wave * 32 + 8 * i4 + 4 * hg]) = v;
      }
      // P slot completed by this step (-1: none, frame scan inside a chunk)
      int slot = dir == 0 ? st + 1 : g.C - 1 - st;
      if (mode == 2) {
        const int f = dir == 0 ? st : g.F - 1 - st;
        slot = dir == 0 ? ((f + 1) % g.cf == 0 ? (f + 1) / g.cf : -1) : (f % g.cf == 0 ? f / g.cf : -1);
      }
      if (Pb && slot >= 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          Pb[(size_t)slot * DD + (size_t)(wave * 32 + mfma32_row(i, hg)) * D + col0 + l32] = acc[i];
      }
      if (out_final && st + 1 == nsteps) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          out_final[(size_t)(wave * 32 + mfma32_row(i, hg)) * D + col0 + l32] = acc[i];
      }
    }
#pragma unroll
    for (int j = 0; j < NK8; ++j) lf[j] = lnext[j];
#pragma unroll
    for (int i = 0; i < 16; ++i) af[i] = anext[i];
  }
  if (out_final && nsteps == 0) {   // single-frame chunk: the map itself
    __syncthreads();
    for (int e = tid; e < D * 32; e += 256) {
      const int k = e / 32, n = e % 32;
      out_final[(size_t)k * D + col0 + n] = Yt[n * YP + k];
    }
  }
}

hipError_t launch_vda_chunk_compose(const Geometry& g, const float* Tf, const float* Uf, float* Tc,
                                    float* Uc, int dirs_mask, hipStream_t s) {
  if (g.D == 64 || g.D == 128) {
    const unsigned grid = (unsigned)(g.B * g.H * 2 * g.C * 2 * (g.D / 32 / kChainG));
    if (g.D == 128)
      vda_chain_mfma_kernel<128><<<grid, 256 * kChainG, 0, s>>>(g, Tf, Uf, Tc, Uc, nullptr, 0.f, nullptr, nullptr, 0, dirs_mask);
    else
      vda_chain_mfma_kernel<64><<<grid, 256 * kChainG, 0, s>>>(g, Tf, Uf, Tc, Uc, nullptr, 0.f, nullptr, nullptr, 0, dirs_mask);
    return hipGetLastError();
  }
  const int NCB = 2 * ((g.D + kCB - 1) / kCB);
  const unsigned grid = (unsigned)(g.B * g.H * 2 * g.C * NCB);
  switch (g.D) {
    case 16: vda_chunk_compose_kernel<16><<<grid, 256, 0, s>>>(g, Tf, Uf, Tc, Uc, dirs_mask); break;
    case 32: vda_chunk_compose_kernel<32><<<grid, 256, 0, s>>>(g, Tf, Uf, Tc, Uc, dirs_mask); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---- prefix scan: grid = B*H * 2 * (D/32 rounded up) ----
template <int D>
__global__ __launch_bounds__(256) void vda_chunk_scan_kernel(Geometry g, const float* __restrict__ Tc,
                                                             const float* __restrict__ Uc,
                                                             const float* __restrict__ S_text,
                                                             float init_scale, float* __restrict__ P_fwd,
                                                             float* __restrict__ P_rev) {
  __shared__ __attribute__((aligned(16))) float smem[D * (D + 1) + 2 * D * kCB];
  float* Ts = smem;
  float* Y0 = smem + D * (D + 1);
  float* Y1 = Y0 + D * kCB;
  constexpr int NCB = (D + kCB - 1) / kCB;
  int id = blockIdx.x;
  const int cb = id % NCB; id /= NCB;
  const int dir = id % 2;
  const int bh = id / 2;
  float* P = dir == 0 ? P_fwd : P_rev;
  if (!P) return;
  const size_t DD = (size_t)D * D;
  const int col0 = cb * kCB;
  const int ncols = min(kCB, D - col0);
  const float* St = S_text + (size_t)bh * DD;
  float* Pb = P + (size_t)bh * (g.C + 1) * DD;
  for (int i = threadIdx.x; i < D * kCB; i += blockDim.x) {
    const int row = i / kCB, col = i % kCB;
    const float v = col < ncols ? init_scale * St[(size_t)row * D + col0 + col] : 0.f;
    Y0[i] = v;
    if (col < ncols) Pb[(size_t)(dir == 0 ? 0 : g.C) * DD + (size_t)row * D + col0 + col] = v;
  }
  float* yin = Y0;
  float* yout = Y1;
  for (int n = 0; n < g.C; ++n) {
    const int c = dir == 0 ? n : g.C - 1 - n;
    const size_t mo = (((size_t)bh * 2 + dir) * g.C + c) * DD;
    __syncthreads();
    stage_matrix<D>(Ts, Tc + mo);
    __syncthreads();
    apply_left<D>(Ts, yin, yout, Uc + mo + col0, D, ncols);
    __syncthreads();
    const int slot = dir == 0 ? c + 1 : c;
    for (int i = threadIdx.x; i < D * kCB; i += blockDim.x) {
      const int row = i / kCB, col = i % kCB;
      if (col < ncols) Pb[(size_t)slot * DD + (size_t)row * D + col0 + col] = yout[i];
    }
    float* t = yin; yin = yout; yout = t;
  }
}

// Frame-level scans straight from the frame maps (D = 64, 128): P_fwd and P_rev
// at the chunk boundaries without composing the chunks first.
hipError_t launch_vda_frame_scan(const Geometry& g, const float* Tf, const float* Uf,
                                 const float* S_text, float init_scale, float* P_fwd, float* P_rev,
                                 hipStream_t s) {
  const int dirs = (P_fwd ? 1 : 0) | (P_rev ? 2 : 0);
  const unsigned grid = (unsigned)(g.B * g.H * 2 * (g.D / 32 / kChainG));
  if (g.D == 128)
    vda_chain_mfma_kernel<128><<<grid, 256 * kChainG, 0, s>>>(g, Tf, Uf, nullptr, nullptr, S_text, init_scale, P_fwd, P_rev, 2, dirs);
  else if (g.D == 64)
    vda_chain_mfma_kernel<64><<<grid, 256 * kChainG, 0, s>>>(g, Tf, Uf, nullptr, nullptr, S_text, init_scale, P_fwd, P_rev, 2, dirs);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_vda_chunk_scan(const Geometry& g, const float* Tc, const float* Uc,
                                 const float* S_text, float init_scale, float* P_fwd, float* P_rev,
                                 hipStream_t s) {
  const int dirs = (P_fwd ? 1 : 0) | (P_rev ? 2 : 0);
  if (g.D == 64 || g.D == 128) {
    const unsigned grid = (unsigned)(g.B * g.H * 2 * (g.D / 32 / kChainG));
    if (g.D == 128)
      vda_chain_mfma_kernel<128><<<grid, 256 * kChainG, 0, s>>>(g, nullptr, nullptr, const_cast<float*>(Tc), const_cast<float*>(Uc), S_text, init_scale, P_fwd, P_rev, 1, dirs);
    else
      vda_chain_mfma_kernel<64><<<grid, 256 * kChainG, 0, s>>>(g, nullptr, nullptr, const_cast<float*>(Tc), const_cast<float*>(Uc), S_text, init_scale, P_fwd, P_rev, 1, dirs);
    return hipGetLastError();
  }
  const int NCB = (g.D + kCB - 1) / kCB;
  const unsigned grid = (unsigned)(g.B * g.H * 2 * NCB);
  switch (g.D) {
    case 16: vda_chunk_scan_kernel<16><<<grid, 256, 0, s>>>(g, Tc, Uc, S_text, init_scale, P_fwd, P_rev); break;
    case 32: vda_chunk_scan_kernel<32><<<grid, 256, 0, s>>>(g, Tc, Uc, S_text, init_scale, P_fwd, P_rev); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace vdn
