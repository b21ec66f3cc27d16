// VDA-Prep: the linear branch's feature map, fused with the layout change.
//
// Paper ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream
// Video Generation"), method, the two branches: the linear branch applies
// its own feature map -- a separable short convolution on K and V made of a
// depthwise spatial filter and a five-tap temporal filter, followed by SiLU,
// with L2 normalisation on Q and K.  System section, fused VDA kernels:
// VDA-Prep fuses the temporal convolution, SiLU, L2 normalisation and the
// conversion to the frame-major layout.
//
//   conv(x)[f,y,x,c] = sum_tau wt[c,tau] sum_{dy,dx} ws[c,dy,dx]
//                      x[f + tau - t0, y + dy - ry, x + dx - rx, c]   (zeros outside)
//   q' = L2(q),  k' = L2(SiLU(conv(k))),  v' = SiLU(conv(v))
//
// Design (HBM-bound: every input element read once from HBM, every output
// written once):
//  - Q: one 8-channel chunk per lane; the D/8 lanes of a (token, head) row
//    reduce the sum of squares with lane shuffles.  Rows are read
//    token-major [B,L,H,d] (all heads of a token adjacent) and written
//    head-major [B,H,L,d].
//  - K, V: one workgroup per (b, h, grid row, tile of XT columns, tensor)
//    slides over the frames.  For each input frame the kernel_h grid rows
//    around the row (with a column halo) are staged in LDS as fp32; each lane
//    task (column, 8 channels) forms the spatial sum for that frame and
//    keeps it in a per-lane circular register window of the last kTapsMax
//    frames (no LDS round trip for the temporal filter).  When the window holds an
//    output frame's last input frame, the temporal sum, SiLU and (for K) the
//    L2 norm over the token's D/8 lanes give the output row, written
//    frame-major.  The next frame's rows are fetched into registers while
//    the current frame is computed.
#include "vdn_common.h"
#include "vdn_internal.h"

#include <type_traits>

namespace vdn {

constexpr int kPrepThreads = 256;

template <typename T> struct Chunk8;
template <> struct Chunk8<bf16_t> {   // 8 bf16 = one 16-byte access
  u32x4 r;
  __device__ __forceinline__ void load(const bf16_t* p) { r = ld16(p); }
  __device__ __forceinline__ void store_raw(bf16_t* p) const { st16(p, r); }
  __device__ __forceinline__ void load_buf(rsrc_t rs, uint32_t off) { r = buf_ld16(rs, off); }
  __device__ __forceinline__ void zero() { r = u32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ void to_f32(float* x) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(r[i] << 16);
      x[2 * i + 1] = __uint_as_float(r[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* x) {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(x[2 * i], x[2 * i + 1]);
    st16(p, o);
  }
};
template <> struct Chunk8<float> {    // 8 float = two 16-byte accesses
  u32x4 r0, r1;
  __device__ __forceinline__ void load(const float* p) { r0 = ld16(p); r1 = ld16(p + 4); }
  __device__ __forceinline__ void store_raw(float* p) const { st16(p, r0); st16(p + 4, r1); }
  __device__ __forceinline__ void load_buf(rsrc_t rs, uint32_t off) {
    r0 = buf_ld16(rs, off);
    r1 = buf_ld16(rs, off + 16);   // an offset past the range stays past it
  }
  __device__ __forceinline__ void zero() { r0 = r1 = u32x4{0, 0, 0, 0}; }
  __device__ __forceinline__ void to_f32(float* x) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = __uint_as_float(r0[i]);
      x[4 + i] = __uint_as_float(r1[i]);
    }
  }
  static __device__ __forceinline__ void store(float* p, const float* x) {
    st16(p, u32x4{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])});
    st16(p + 4, u32x4{__float_as_uint(x[4]), __float_as_uint(x[5]), __float_as_uint(x[6]), __float_as_uint(x[7])});
  }
};

// SiLU with a hardware reciprocal (about 1 ulp): x -> -inf gives -0.
__device__ __forceinline__ float silu(float x) { return x * __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// Sum over the `lanes` consecutive lanes (a power of two <= 16) of one row.
__device__ __forceinline__ float row_sum(float x, int lanes) {
  for (int off = lanes >> 1; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// ---------------------------------------------------------------------------
// Q: L2 normalisation + [B,L,H,d] -> [B,H,L,d].
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kPrepThreads) void vda_prep_q_kernel(const T* __restrict__ q,
                                                                   T* __restrict__ q_out,
                                                                   long long rows, int H,
                                                                   long long L, float eps) {
  constexpr int C8 = D / 8;
  const long long row = ((long long)blockIdx.x * kPrepThreads + threadIdx.x) / C8;   // (b, l, h)
  const int c8 = threadIdx.x % C8;
  const bool ok = row < rows;
  float x[8] = {};
  if (ok) {
    Chunk8<T> c;
    c.load(q + (size_t)row * D + c8 * 8);
    c.to_f32(x);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss = fmaf(x[i], x[i], ss);
  ss = row_sum(ss, C8);
  if (!ok) return;
  const float r = rsqrtf(ss + eps);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] *= r;
  const int h = (int)(row % H);
  const long long bl = row / H, b = bl / L, l = bl % L;
  Chunk8<T>::store(q_out + (((size_t)b * H + h) * L + l) * D + c8 * 8, x);
}

// ---------------------------------------------------------------------------
// K, V: separable short convolution + SiLU (+ L2 for K) + layout change.
// ---------------------------------------------------------------------------
constexpr int kTapsMax = 5;
constexpr int kRing = 5;          // register window slots
constexpr int kPrefetchMax = 8;   // staged 8-channel chunks per thread and frame

struct PrepArgs {
  const void* src[2];     // k, v   [B,L,H,D]
  void* dst[2];           // k', v' [B,H,L,D]
  const float* w_sp;      // [H,D,kh,kw]
  const float* w_t;       // [H,D,taps]
  int B, H, F, gh, gw, kh, kw, taps, t0, xt, ntx;
  long long L;
  float eps;
};

// KH, KW > 0 fix the spatial filter size at compile time (fully unrolled
// taps); 0 reads it from the arguments.
template <typename T, int D, int KH, int KW>
__global__ __launch_bounds__(kPrepThreads) void vda_prep_kv_kernel(PrepArgs a) {
  constexpr int C8 = D / 8;
  const int kh = KH > 0 ? KH : a.kh, kw = KW > 0 ? KW : a.kw;
  constexpr int TPT = (16 * C8 + kPrepThreads - 1) / kPrepThreads;   // column-pair tasks per thread (xt <= 32)
  extern __shared__ __attribute__((aligned(16))) float sm[];
  // LDS: spatial weights [kh*kw][D] | temporal weights by window slot
  // [kTapsMax][D] | staged rows [kh][xt + kw - 1][D], kept in the storage
  // type (the spatial sums convert to fp32 as they read)
  const int cols = a.xt + kw - 1;
  float* ws_s = sm;
  float* wt_s = ws_s + (size_t)kh * kw * D;
  T* in_s = reinterpret_cast<T*>(wt_s + (size_t)kTapsMax * D);

  // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs, so XCD
  // x = blockIdx % 8 takes a contiguous run of the logical order (b, h,
  // tensor, grid row, column tile); workgroups of neighbouring grid rows,
  // which stage the same input rows, then share that XCD's L2.
  const int total = a.B * a.H * 2 * a.gh * a.ntx;
  const int per = (total + kNumXcd - 1) / kNumXcd;
  int bid = (int)(blockIdx.x % kNumXcd) * per + (int)(blockIdx.x / kNumXcd);
  if (bid >= total) return;
  const int xt_i = bid % a.ntx; bid /= a.ntx;
  const int y = bid % a.gh; bid /= a.gh;
  const int which = bid & 1; bid >>= 1;             // 0 = K, 1 = V
  const int h = bid % a.H;
  const int b = bid / a.H;
  const int x0 = xt_i * a.xt;
  const T* src = static_cast<const T*>(a.src[which]);
  T* dst = static_cast<T*>(a.dst[which]);
  const int tid = threadIdx.x;
  const int N = a.gh * a.gw;
  const int ry = (kh - 1) / 2, rx = (kw - 1) / 2;

  // filters of head h: spatial [tap][c]; temporal placed at the window slots
  // kTapsMax - taps .. kTapsMax - 1 (older slots get zero)
  for (int e = tid; e < kh * kw * D; e += kPrepThreads) {
    const int tap = e / D, c = e % D;
    ws_s[e] = a.w_sp[((size_t)h * D + c) * kh * kw + tap];
  }
  for (int e = tid; e < kTapsMax * D; e += kPrepThreads) {
    const int slot = e / D, c = e % D;
    const int tap = slot - (kTapsMax - a.taps);
    wt_s[e] = tap >= 0 ? a.w_t[((size_t)h * D + c) * a.taps + tap] : 0.f;
  }

  // staging: chunk q -> (row r, column cx, c8), at a fixed byte offset from
  // the start of a frame's rows of head h; chunks outside the grid (and
  // past the staged block) get an offset beyond the buffer range, which
  // reads as zeros, so the frame loop carries no index arithmetic or
  // bounds branches
  const int nchunk = kh * cols * C8;
  uint32_t coff[kPrefetchMax];
#pragma unroll
  for (int i = 0; i < kPrefetchMax; ++i) {
    const int qq = tid + kPrepThreads * i;
    coff[i] = 0x80000000u;
    if (qq < nchunk) {
      const int c8 = qq % C8, rc = qq / C8;
      const int cx = rc % cols, r = rc / cols;
      const int yy = y + r - ry, xx = x0 + cx - rx;
      if (yy >= 0 && yy < a.gh && xx >= 0 && xx < a.gw)
        coff[i] = (uint32_t)((((size_t)yy * a.gw + xx) * a.H * D + c8 * 8) * sizeof(T));
    }
  }
  const size_t frame_elems = (size_t)N * a.H * D;
  const T* hbase = src + (size_t)b * a.L * a.H * D + (size_t)h * D;
  const T* tend = src + (size_t)a.B * a.L * a.H * D;
  Chunk8<T> pf[kPrefetchMax];   // next frame's rows, fetched one frame ahead
  auto fetch = [&](Chunk8<T>* pf, int fi) {
    if (fi < a.F) {
      const T* fb = hbase + (size_t)fi * frame_elems;
      const rsrc_t rs = make_rsrc(fb, rsrc_bytes(fb, tend));
#pragma unroll
      for (int i = 0; i < kPrefetchMax; ++i) pf[i].load_buf(rs, coff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < kPrefetchMax; ++i) pf[i].zero();
    }
  };
  auto stage = [&](const Chunk8<T>* pf) {
#pragma unroll
    for (int i = 0; i < kPrefetchMax; ++i) {
      const int qq = tid + kPrepThreads * i;
      if (qq < nchunk) pf[i].store_raw(in_s + (size_t)qq * 8);   // = row (qq / C8), channels 8 (qq % C8)
    }
  };

  // spatial sums of recent frames in a circular window: frame fi lives in
  // slot fi % kRing, so the frame loop is unrolled kRing times and every slot
  // index is static (no register shuffling).  A lane task covers two
  // adjacent columns, which share kw of their kw + 1 input columns.
  float win[TPT][kRing][2][8];
#pragma unroll
  for (int j = 0; j < TPT; ++j)
#pragma unroll
    for (int sl = 0; sl < kRing; ++sl)
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 8; ++i) win[j][sl][e][i] = 0.f;

  constexpr int KWM = KW > 0 ? KW : 7, KHM = KH > 0 ? KH : 7;
  const int nsteps = a.F + a.taps - 1 - a.t0;
  auto step = [&](int fi, auto uc) {
    constexpr int u = decltype(uc)::value;   // = fi % kRing
    __syncthreads();     // previous frame's spatial reads done; filters staged
    stage(pf);
    __syncthreads();
    if (fi + 1 < nsteps) fetch(pf, fi + 1);
    const int fo = fi - (a.taps - 1 - a.t0);
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int t = tid + kPrepThreads * j;
      const int xl = 2 * (t / C8), c8 = t % C8;
      const bool act[2] = {xl < a.xt && x0 + xl < a.gw, xl + 1 < a.xt && x0 + xl + 1 < a.gw};
      // the first tap of each sum multiplies (no zero-initialised accumulators)
      float s[2][8];
      if (act[0]) {
#pragma unroll
        for (int dy = 0; dy < KHM; ++dy) {
          if (KH == 0 && dy >= kh) continue;
          float xc[KWM + 1][8];
#pragma unroll
          for (int cx = 0; cx <= KWM; ++cx) {
            if (KW == 0 && cx > kw) continue;
            Chunk8<T> xin;
            xin.load(in_s + (size_t)(dy * cols + xl + cx) * D + c8 * 8);
            xin.to_f32(xc[cx]);
          }
#pragma unroll
          for (int dx = 0; dx < KWM; ++dx) {
            if (KW == 0 && dx >= kw) continue;
            const float* w = ws_s + (size_t)(dy * kw + dx) * D + c8 * 8;
            const u32x4 w0v = ld16(w), w1v = ld16(w + 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float wa = __uint_as_float(w0v[i]), wb = __uint_as_float(w1v[i]);
              if (dy == 0 && dx == 0) {
                s[0][i] = wa * xc[dx][i];
                s[0][4 + i] = wb * xc[dx][4 + i];
                s[1][i] = wa * xc[dx + 1][i];
                s[1][4 + i] = wb * xc[dx + 1][4 + i];
              } else {
                s[0][i] = fmaf(wa, xc[dx][i], s[0][i]);
                s[0][4 + i] = fmaf(wb, xc[dx][4 + i], s[0][4 + i]);
                s[1][i] = fmaf(wa, xc[dx + 1][i], s[1][i]);
                s[1][4 + i] = fmaf(wb, xc[dx + 1][4 + i], s[1][4 + i]);
              }
            }
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int i = 0; i < 8; ++i) s[e][i] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int i = 0; i < 8; ++i) win[j][u][e][i] = s[e][i];
      if (fo < 0) continue;
      // frame fi - k (slot (u - k) mod kRing) meets temporal weight slot kTapsMax - 1 - k
      float o[2][8];
#pragma unroll
      for (int k = 0; k < kTapsMax; ++k) {
        const int sl = (u - k + kRing) % kRing;
        const float* w = wt_s + (size_t)(kTapsMax - 1 - k) * D + c8 * 8;
        const u32x4 w0v = ld16(w), w1v = ld16(w + 4);
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float wa = __uint_as_float(w0v[i]), wb = __uint_as_float(w1v[i]);
            o[e][i] = k == 0 ? wa * win[j][sl][e][i] : fmaf(wa, win[j][sl][e][i], o[e][i]);
            o[e][4 + i] = k == 0 ? wb * win[j][sl][e][4 + i] : fmaf(wb, win[j][sl][e][4 + i], o[e][4 + i]);
          }
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
#pragma unroll
        for (int i = 0; i < 8; ++i) o[e][i] = silu(o[e][i]);
        if (which == 0) {   // K: L2 over the token's D channels (its C8 consecutive lanes)
          float ss = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) ss = fmaf(o[e][i], o[e][i], ss);
          ss = row_sum(ss, C8);
          const float r = rsqrtf(ss + a.eps);
#pragma unroll
          for (int i = 0; i < 8; ++i) o[e][i] *= r;
        }
        if (act[e]) {
          const long long l = (long long)fo * N + (long long)y * a.gw + x0 + xl + e;
          Chunk8<T>::store(dst + (((size_t)b * a.H + h) * a.L + l) * D + c8 * 8, o[e]);
        }
      }
    }
  };
  fetch(pf, 0);
  for (int fb = 0; fb < nsteps; fb += kRing) {
    step(fb, std::integral_constant<int, 0>{});
    if (fb + 1 < nsteps) step(fb + 1, std::integral_constant<int, 1>{});
    if (fb + 2 < nsteps) step(fb + 2, std::integral_constant<int, 2>{});
    if (fb + 3 < nsteps) step(fb + 3, std::integral_constant<int, 3>{});
    if (fb + 4 < nsteps) step(fb + 4, std::integral_constant<int, 4>{});
  }
  static_assert(kRing == 5 && kRing >= kTapsMax, "the frame loop is unrolled kRing times");
}

// Largest even column tile (<= 32) whose LDS footprint stays within 64 KB
// with the rows staged as fp32 (bf16 rows take less);
// a grid narrower than the tile rounds up to even (the extra column is
// outside the grid and reads as zeros).
int prep_tile_cols(int D, int kh, int kw, int gw) {
  for (int xt = 32; xt >= 2; xt >>= 1) {
    const size_t bytes = ((size_t)kh * (xt + kw - 1) * D + (size_t)kh * kw * D + (size_t)kTapsMax * D) * 4;
    const int chunks = kh * (xt + kw - 1) * (D / 8);
    if (bytes <= 65536 && chunks <= kPrefetchMax * kPrepThreads) return xt < gw ? xt : (gw + 1) / 2 * 2;
  }
  return 0;
}

template <typename T>
hipError_t launch_vda_prep(const void* q, const void* k, const void* v, const float* w_sp,
                           const float* w_t, void* q_out, void* k_out, void* v_out, int B, int H,
                           int F, int gh, int gw, int D, int kh, int kw, int taps, int causal,
                           float eps, hipStream_t s) {
  const long long L = (long long)F * gh * gw;
  const long long rows = (long long)B * L * H;
  const long long qthreads = rows * (D / 8);
  const unsigned qgrid = (unsigned)((qthreads + kPrepThreads - 1) / kPrepThreads);
  PrepArgs a;
  a.src[0] = k; a.src[1] = v; a.dst[0] = k_out; a.dst[1] = v_out;
  a.w_sp = w_sp; a.w_t = w_t;
  a.B = B; a.H = H; a.F = F; a.gh = gh; a.gw = gw; a.kh = kh; a.kw = kw; a.taps = taps;
  a.t0 = causal ? taps - 1 : (taps - 1) / 2;
  a.xt = prep_tile_cols(D, kh, kw, gw);
  if (a.xt <= 0) return hipErrorInvalidValue;
  a.ntx = (gw + a.xt - 1) / a.xt;
  a.L = L;
  a.eps = eps;
  const long long kvtotal = (long long)B * H * gh * a.ntx * 2;
  const unsigned kvgrid = (unsigned)((kvtotal + kNumXcd - 1) / kNumXcd * kNumXcd);
  const size_t lds = (size_t)kh * (a.xt + kw - 1) * D * sizeof(T) + ((size_t)kh * kw * D + (size_t)kTapsMax * D) * 4;
#define VDN_PREP_CASE(DD)                                                                          \
  case DD:                                                                                         \
    vda_prep_q_kernel<T, DD><<<qgrid, kPrepThreads, 0, s>>>((const T*)q, (T*)q_out, rows, H, L, eps); \
    if (kh == 3 && kw == 3)                                                                        \
      vda_prep_kv_kernel<T, DD, 3, 3><<<kvgrid, kPrepThreads, lds, s>>>(a);                        \
    else                                                                                           \
      vda_prep_kv_kernel<T, DD, 0, 0><<<kvgrid, kPrepThreads, lds, s>>>(a);                        \
    break;
  switch (D) {
    VDN_PREP_CASE(16)
    VDN_PREP_CASE(32)
    VDN_PREP_CASE(64)
    VDN_PREP_CASE(128)
    default: return hipErrorInvalidValue;
  }
#undef VDN_PREP_CASE
  return hipGetLastError();
}

template hipError_t launch_vda_prep<bf16_t>(const void*, const void*, const void*, const float*,
                                            const float*, void*, void*, void*, int, int, int, int,
                                            int, int, int, int, int, int, float, hipStream_t);
template hipError_t launch_vda_prep<float>(const void*, const void*, const void*, const float*,
                                           const float*, void*, void*, void*, int, int, int, int,
                                           int, int, int, int, int, int, float, hipStream_t);

}  // namespace vdn
