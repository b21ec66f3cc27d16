// Gated merge of the two branches through separate output projections.
//
// Paper ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream
// Video Generation"), method, branch calibration: each branch has its own
// output projection and the two projected outputs are added, so
//   out[M, Dm] = Ohat_s[M, K] W_s[K, Dm] + Ohat_l[M, K] W_l[K, Dm]
// with M = B*L tokens and K = H*d_v (heads concatenated).  This is one GEMM
// over the concatenated contraction [Ohat_s | Ohat_l] [W_s ; W_l].
//
// bf16 path: both operands K-contiguous (the projections are transposed
// once per call into the workspace, W^T [Dm, K]), 256 x 256 output tiles,
// 64-deep K steps through double-buffered LDS with the next steps' global
// loads in flight, v_mfma_f32_32x32x16_bf16 with fp32 accumulation.  The
// product is formed as out^T blocks (each lane owns 4 consecutive output
// features of one token); the finished tile is written through LDS as whole
// row segments.
#include "vdn_common.h"
#include "vdn_internal.h"
#include "gemm_nt.h"

namespace vdn {

constexpr int kGBM = 256, kGBN = 256, kGBK = 64;
constexpr int kGroupRows = 4;
// 8 waves (two per SIMD): wave (wm 0..3, wn 0..1) owns a 64 x 128 block of
// the 256 x 256 tile.  Operand panels are read with buffer loads whose
// descriptors end at the last row of A / W^T, so rows past M or N read as
// zero without branches; K must be a multiple of the 64-deep K step.  The
// LDS fragments of the next 16-deep step are loaded while the current
// step's MFMAs run, and each 16-deep step stores one 16-byte chunk per
// operand of the next K step to LDS and requests the same chunk of the one
// after, so vector-memory requests are spread over the K step (scheduling
// barriers keep the compiler from regrouping them).  One LDS-only barrier
// per K step.
//
// Tile order: XCD x (blockIdx % 8) owns a contiguous range of row tiles and
// walks it in groups of kGroupRows rows, column by column inside a group, so
// the workgroups resident on one XCD share A row panels and W^T column
// panels in that XCD's L2.
//
// LD = false: the operands are packed (row pitch K).  LD = true: rows of all
// four operands have pitch ld >= K, which lets one product with a
// contraction of 2K be split into two halves of the same rows (a1 = a0 + K,
// bt1 = bt0 + K, ld = 2K): the backward's GEMMs.
template <bool LD>
__global__ __launch_bounds__(512) void merge_gemm_bf16_kernel(const bf16_t* __restrict__ a0,
                                                              const bf16_t* __restrict__ a1,
                                                              const bf16_t* __restrict__ bt0,
                                                              const bf16_t* __restrict__ bt1,
                                                              bf16_t* __restrict__ out,
                                                              long long M, int K, int N,
                                                              int tiles_m, int tiles_n, int rpx,
                                                              long long ld_) {
  constexpr int BM = kGBM, BN = kGBN, BK = kGBK;
  constexpr int P = BK + 8;
  constexpr int CH = BM * BK / 8 / 512;   // 16-byte chunks per thread per operand and K step (4)
  constexpr int NSUB = BK / 16;           // 16-deep MFMA steps per K step (4)
  static_assert(CH == NSUB, "one chunk of each operand staged per MFMA step");
  // buffer b: the A panel, then the W^T panel; after the K loop the whole
  // array holds the output tile
  __shared__ __attribute__((aligned(16))) bf16_t lds[2][(BM + BN) * P];
  auto As = [&](int b) { return &lds[b][0]; };
  auto Bs = [&](int b) { return &lds[b][BM * P]; };
  // XCD-aware grouped order: XCD x owns row tiles [x rpx, (x+1) rpx) and walks
  // them in groups of kGroupRows rows, column by column inside a group.
  const int x = blockIdx.x % kNumXcd;
  const int t = blockIdx.x / kNumXcd;
  const int gsz = kGroupRows * tiles_n;
  const int grp = t / gsz, rem = t % gsz;
  const int col = rem / kGroupRows;
  const int row = x * rpx + grp * kGroupRows + rem % kGroupRows;
  const int row_end = min((x + 1) * rpx, tiles_m);
  if (row >= row_end) return;
  const long long m0 = (long long)row * BM;
  const int n0 = col * BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hg = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;
  const int nkt = 2 * K / BK;   // K % BK == 0
  // row pitch; each descriptor ends at the end of its operand's last row
  const size_t ld = LD ? (size_t)ld_ : (size_t)K;
  const size_t ea = (size_t)(M - 1) * ld + K, eb = (size_t)(N - 1) * ld + K;
  const rsrc_t ra0 = make_rsrc(a0 + (size_t)m0 * ld, rsrc_bytes(a0 + (size_t)m0 * ld, a0 + ea));
  const rsrc_t ra1 = make_rsrc(a1 + (size_t)m0 * ld, rsrc_bytes(a1 + (size_t)m0 * ld, a1 + ea));
  const rsrc_t rb0 = make_rsrc(bt0 + (size_t)n0 * ld, rsrc_bytes(bt0 + (size_t)n0 * ld, bt0 + eb));
  const rsrc_t rb1 = make_rsrc(bt1 + (size_t)n0 * ld, rsrc_bytes(bt1 + (size_t)n0 * ld, bt1 + eb));
  uint32_t voff[CH];
  int soff[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + 512 * i;
    const int r = c / (BK / 8), c8 = c % (BK / 8);
    voff[i] = (uint32_t)((r * ld + c8 * 8) * 2);
    soff[i] = (r * P + c8 * 8);
  }
  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};
  u32x4 pa[CH], pb[CH];
  auto load_piece = [&](int i, int kt) {   // K steps past the end re-read the last one
    kt = min(kt, nkt - 1);
    const int k0 = kt * BK;
    const bool second = k0 >= K;
    const uint32_t kb = (uint32_t)((second ? k0 - K : k0) * 2);
    pa[i] = buf_ld16(second ? ra1 : ra0, voff[i], kb);
    pb[i] = buf_ld16(second ? rb1 : rb0, voff[i], kb);
  };
  auto store_piece = [&](int i, int buf) {
    st16(As(buf) + soff[i], pa[i]);
    st16(Bs(buf) + soff[i], pb[i]);
  };
#pragma unroll
  for (int i = 0; i < CH; ++i) load_piece(i, 0);
#pragma unroll
  for (int i = 0; i < CH; ++i) store_piece(i, 0);
#pragma unroll
  for (int i = 0; i < CH; ++i) load_piece(i, 1);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const bf16_t* Ab = As(kt & 1) + (wm * 64 + l32) * P + hg * 8;
    const bf16_t* Bb = Bs(kt & 1) + (wn * 128 + l32) * P + hg * 8;
    bf16x8 fm[2][2], fn[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i) fm[0][i] = as_bf16x8(ld16(Ab + i * 32 * P));
#pragma unroll
    for (int i = 0; i < 4; ++i) fn[0][i] = as_bf16x8(ld16(Bb + i * 32 * P));
#pragma unroll
    for (int ks = 0; ks < NSUB; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;
      if (ks + 1 < NSUB) {
#pragma unroll
        for (int i = 0; i < 2; ++i) fm[nxt][i] = as_bf16x8(ld16(Ab + i * 32 * P + (ks + 1) * 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) fn[nxt][i] = as_bf16x8(ld16(Bb + i * 32 * P + (ks + 1) * 16));
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc[nb][mb] = mfma32x32x16(fn[cur][nb], fm[cur][mb], acc[nb][mb]);
      // stage chunk ks of the next K step, request it for the one after
      store_piece(ks, (kt + 1) & 1);
      load_piece(ks, kt + 2);
      // issue order: each of the next step's six fragment reads after one
      // MFMA, then the LDS stores and the global loads between the last two
      if (ks + 1 < NSUB) {
#pragma unroll
        for (int u = 0; u < 6; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);       // 2 LDS writes
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);       // 2 global loads
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();
  }
  // Epilogue: the 256 x 256 tile goes through LDS (the operand buffers are
  // free after the K loop) and leaves as 512-byte row segments, 16 bytes per
  // lane: from the MFMA layout each store would write 8 bytes into each of
  // 32 rows D * 2 bytes apart.
  constexpr int TP = BN + 8;   // tile pitch (bf16)
  static_assert(BM * TP <= 2 * (BM + BN) * P, "output tile fits in the operand buffers");
  bf16_t* tile = &lds[0][0];
  __syncthreads();             // every wave is done with the operand tiles
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[nb][mb][i4 * 4 + 0], acc[nb][mb][i4 * 4 + 1]);
        pk[1] = pack_bf16x2(acc[nb][mb][i4 * 4 + 2], acc[nb][mb][i4 * 4 + 3]);
        *reinterpret_cast<u32x2*>(&tile[(wm * 64 + mb * 32 + l32) * TP + wn * 128 + nb * 32 + 8 * i4 + 4 * hg]) = pk;
      }
  __syncthreads();
  const int c8 = (tid % (BN / 8)) * 8;
  const bool col_ok = n0 + c8 < N;   // N % 8 == 0
#pragma unroll 4
  for (int it = 0; it < BM * (BN / 8) / 512; ++it) {
    const int r = it * (512 / (BN / 8)) + tid / (BN / 8);
    const long long m = m0 + r;
    const u32x4 v = ld16(&tile[r * TP + c8]);
    if (m < M && col_ok) st16(out + (size_t)m * N + n0 + c8, v);
  }
}

hipError_t launch_merge_gemm_bf16(const uint16_t* a0, const uint16_t* a1, const uint16_t* w0t,
                                  const uint16_t* w1t, uint16_t* out, long long M, int K, int Dm,
                                  hipStream_t s) {
  if (M == 0 || Dm == 0) return hipSuccess;
  if (Dm % 8 != 0) return hipErrorInvalidValue;   // 16-byte output rows
  const int tm = (int)((M + kGBM - 1) / kGBM), tn = (Dm + kGBN - 1) / kGBN;
  const int rpx = (tm + kNumXcd - 1) / kNumXcd;
  const int groups = (rpx + kGroupRows - 1) / kGroupRows;
  const long long grid = (long long)kNumXcd * groups * kGroupRows * tn;
  merge_gemm_bf16_kernel<false><<<(unsigned)grid, 512, 0, s>>>(a0, a1, w0t, w1t, out, M, K, Dm, tm,
                                                               tn, rpx, 0);
  return hipGetLastError();
}

hipError_t launch_gemm_nt_bf16(const uint16_t* a, const uint16_t* bt, uint16_t* out, long long M,
                               long long Kc, int N, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (N % 8 != 0) return hipErrorInvalidValue;   // 16-byte output rows
  if (Kc % (2 * kGBK) != 0 || Kc / 2 > 0x7FFFFFFF) return hipErrorInvalidValue;
  const int K = (int)(Kc / 2);
  const int tm = (int)((M + kGBM - 1) / kGBM), tn = (N + kGBN - 1) / kGBN;
  const int rpx = (tm + kNumXcd - 1) / kNumXcd;
  const int groups = (rpx + kGroupRows - 1) / kGroupRows;
  const long long grid = (long long)kNumXcd * groups * kGroupRows * tn;
  merge_gemm_bf16_kernel<true><<<(unsigned)grid, 512, 0, s>>>(a, a + K, bt, bt + K, out, M, K, N, tm,
                                                              tn, rpx, Kc);
  return hipGetLastError();
}
// ---- generic SIMT GEMM (fp32 storage or odd shapes): 16x16 tiles ----
template <typename T>
__global__ __launch_bounds__(256) void merge_gemm_simt_kernel(const T* __restrict__ a0,
                                                              const T* __restrict__ a1,
                                                              const T* __restrict__ w0,
                                                              const T* __restrict__ w1,
                                                              T* __restrict__ out, long long M,
                                                              int K, int N) {
  __shared__ float As[16][17];
  __shared__ float Ws[16][17];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const long long m = (long long)blockIdx.y * 16 + ty;
  const int n = blockIdx.x * 16 + tx;
  float acc = 0.f;
  for (int part = 0; part < 2; ++part) {
    const T* a = part ? a1 : a0;
    const T* w = part ? w1 : w0;
    for (int k0 = 0; k0 < K; k0 += 16) {
      __syncthreads();
      const long long am = (long long)blockIdx.y * 16 + ty;
      As[ty][tx] = (am < M && k0 + tx < K) ? Elem<T>::load(a, (size_t)am * K + k0 + tx) : 0.f;
      Ws[ty][tx] = (k0 + ty < K && n < N) ? Elem<T>::load(w, (size_t)(k0 + ty) * N + n) : 0.f;
      __syncthreads();
#pragma unroll
      for (int k = 0; k < 16; ++k) acc = fmaf(As[ty][k], Ws[k][tx], acc);
    }
  }
  if (m < M && n < N) Elem<T>::store(out, (size_t)m * N + n, acc);
}

template <typename T>
hipError_t launch_merge_gemm_simt(const T* a0, const T* a1, const T* w0, const T* w1, T* out,
                                  long long M, int K, int Dm, hipStream_t s) {
  if (M == 0 || Dm == 0) return hipSuccess;
  dim3 grid((unsigned)((Dm + 15) / 16), (unsigned)((M + 15) / 16));
  merge_gemm_simt_kernel<T><<<grid, 256, 0, s>>>(a0, a1, w0, w1, out, M, K, Dm);
  return hipGetLastError();
}

template <typename T>
__global__ void add_kernel(const T* __restrict__ a, const T* __restrict__ b, T* __restrict__ out,
                           long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) Elem<T>::store(out, i, Elem<T>::load(a, i) + Elem<T>::load(b, i));
}

template <typename T>
hipError_t launch_add(const T* a, const T* b, T* out, long long n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  add_kernel<T><<<(unsigned)((n + 255) / 256), 256, 0, s>>>(a, b, out, n);
  return hipGetLastError();
}

template hipError_t launch_merge_gemm_simt<float>(const float*, const float*, const float*,
                                                  const float*, float*, long long, int, int,
                                                  hipStream_t);
template hipError_t launch_merge_gemm_simt<bf16_t>(const bf16_t*, const bf16_t*, const bf16_t*,
                                                   const bf16_t*, bf16_t*, long long, int, int,
                                                   hipStream_t);
template hipError_t launch_add<float>(const float*, const float*, float*, long long, hipStream_t);
template hipError_t launch_add<bf16_t>(const bf16_t*, const bf16_t*, bf16_t*, long long, hipStream_t);

}  // namespace vdn
