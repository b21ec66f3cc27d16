// MX-FP8 merge of the two branches.
//
// Paper ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream
// Video Generation"), system section, other optimizations: the wide output
// GEMMs run in MXFP8 while recurrent states and small-matrix inverses stay in
// FP32.  Here that is out = [Ohat_s | Ohat_l] [W_s ; W_l] with both operands
// in the OCP Microscaling (MX) v1.0 format: blocks of 32 consecutive
// elements along the contraction index share a power-of-two scale (an E8M0
// byte), elements are FP8 E4M3.  Scale of a block: 2^(floor(log2 amax) - 8),
// clamped to [2^-127, 2^127]; element: v / scale rounded to nearest even,
// magnitudes from 448 up saturating to 448.
//
// Quantizer: one thread per 32-element block of a bf16 row; the row may be
// written at a column offset, so Ohat_s and Ohat_l fill the two halves of
// one [M, 2K] operand.
//
// GEMM: v_mfma_scale_f32_32x32x64_f8f6f4 with fp32 accumulation, 256 x 256
// output tiles, 128-byte (128-element) K steps through double-buffered LDS,
// the same staging, XCD-grouped tile order and out^T store layout as the
// bf16 merge GEMM.  Operand layout of the instruction (fp8 operands, wave64):
// lane l supplies row l % 32; its 32 bytes are the elements 16 h .. 16 h + 15
// and 32 + 16 h .. 32 + 16 h + 15 of the 64-deep step (h = l / 32); its
// scale register supplies, in the byte chosen by op_sel, the scale of block
// h of that step for its row.  A lane's scale dword therefore holds the four
// block scales of its row for one 128-deep K step, shifted right by 8 h so
// that op_sel 0 / 2 selects blocks h / 2 + h.
#include "vdn_common.h"
#include "vdn_internal.h"

namespace vdn {

// fp32 -> E4M3 code: round to nearest even, saturate at 448, keep the sign.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sgn = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t c;
  if (a >= 0x43E00000u) {            // |y| >= 448
    c = 0x7Eu;
  } else if (a >= 0x3C800000u) {     // |y| >= 2^-6: normal, keep 3 mantissa bits
    const uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    c = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);
  } else {                           // subnormal: a multiple of 2^-9 (8 is the smallest normal)
    c = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.f);
  }
  return sgn | c;
}

// Shared exponent of a block whose largest magnitude is amax.
__device__ __forceinline__ int mx_shared_exp(float amax) {
  if (!(amax > 0.f)) return -127;
  int e;
  (void)frexpf(amax, &e);            // amax = f 2^e, f in [0.5, 1)
  const int s = e - 1 - 8;
  return s < -127 ? -127 : (s > 127 ? 127 : s);
}

__global__ __launch_bounds__(256) void mx_quant_rows_kernel(const bf16_t* __restrict__ src,
                                                            long long rows, int cols,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales,
                                                            long long dst_ld, int dst_col0) {
  const int nb = cols / 32;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= rows * nb) return;
  const long long row = gid / nb;
  const int blk = (int)(gid % nb);
  const bf16_t* s = src + (size_t)row * cols + blk * 32;
  u32x4 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = ld16(s + 8 * i);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(__uint_as_float(v[i][j] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(v[i][j] & 0xFFFF0000u)));
    }
  const int se = mx_shared_exp(amax);
  u32x4 out[2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = e4m3_code(ldexpf(__uint_as_float(v[i][j] << 16), -se));
      const uint32_t hi = e4m3_code(ldexpf(__uint_as_float(v[i][j] & 0xFFFF0000u), -se));
      const int byte = 8 * i + 2 * j;            // element index in the block
      const uint32_t pair = lo | (hi << 8);
      if ((byte & 2) == 0)
        out[byte >> 4][(byte >> 2) & 3] = pair;
      else
        out[byte >> 4][(byte >> 2) & 3] |= pair << 16;
    }
  uint8_t* d = codes + (size_t)row * dst_ld + dst_col0 + blk * 32;
  st16(d, out[0]);
  st16(d + 16, out[1]);
  scales[(size_t)row * (dst_ld / 32) + dst_col0 / 32 + blk] = (uint8_t)(se + 127);
}

hipError_t launch_mx_quant_rows(const uint16_t* src, long long rows, int cols, uint8_t* codes,
                                uint8_t* scales, long long dst_ld, int dst_col0, hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (cols % 32 || dst_ld % 32 || dst_col0 % 32 || dst_col0 + cols > dst_ld) return hipErrorInvalidValue;
  const long long n = rows * (cols / 32);
  mx_quant_rows_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(src, rows, cols, codes, scales,
                                                                   dst_ld, dst_col0);
  return hipGetLastError();
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kMxBM = 256, kMxBN = 256, kMxBK = 128;   // BK in elements (= bytes)
constexpr int kMxGroupRows = 4;

template <int OPSEL>
__device__ __forceinline__ f32x16 mfma_mx(const i32x8& a, const i32x8& b, f32x16 c, int sa, int sb) {
  // first operand: rows of the result; formats 0 / 0 = fp8 E4M3
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPSEL, sa, OPSEL, sb);
}

// 4 waves (one per SIMD): wave (wm 0..1, wn 0..1) owns a 128 x 128 block of
// the 256 x 256 tile (16 accumulator blocks), computed as out^T blocks (W^T
// rows are the MFMA's first operand), so each fragment read from LDS feeds
// four MFMAs; the next 64-deep step's fragments are read while the current
// step's MFMAs run.  K2 (the concatenated contraction) is a multiple of 128.
__global__ __launch_bounds__(256) void merge_gemm_mx_kernel(const uint8_t* __restrict__ a,
                                                            const uint8_t* __restrict__ a_sc,
                                                            const uint8_t* __restrict__ bt,
                                                            const uint8_t* __restrict__ b_sc,
                                                            bf16_t* __restrict__ out, long long M,
                                                            int K2, int N, int tiles_m,
                                                            int tiles_n, int rpx) {
  constexpr int BM = kMxBM, BN = kMxBN, BK = kMxBK;
  constexpr int P = BK + 16;                 // LDS row pitch in bytes
  constexpr int CH = BM * BK / 16 / 256;     // 16-byte chunks per thread per operand and K step (8)
  constexpr int NSUB = BK / 64;              // 64-deep MFMA steps per K step (2)
  constexpr int CPS = CH / NSUB;             // chunks per operand staged per MFMA step (2)
  // buffer b: the A panel, then the W^T panel; after the K loop the whole
  // array holds the bf16 output tile
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * P];
  auto As = [&](int b) { return &lds[b][0]; };
  auto Bs = [&](int b) { return &lds[b][BM * P]; };
  const int x = blockIdx.x % kNumXcd;
  const int t = blockIdx.x / kNumXcd;
  const int gsz = kMxGroupRows * tiles_n;
  const int grp = t / gsz, rem = t % gsz;
  const int col = rem / kMxGroupRows;
  const int row = x * rpx + grp * kMxGroupRows + rem % kMxGroupRows;
  const int row_end = min((x + 1) * rpx, tiles_m);
  if (row >= row_end) return;
  const long long m0 = (long long)row * BM;
  const int n0 = col * BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hg = lane >> 5, l32 = lane & 31;
  const int wm = wave >> 1, wn = wave & 1;   // 4 waves, each 128 x 128
  const int nkt = K2 / BK;
  const int nsc = K2 / 32;                   // scale bytes per row
  const rsrc_t ra = make_rsrc(a + (size_t)m0 * K2, rsrc_bytes(a + (size_t)m0 * K2, a + (size_t)M * K2));
  const rsrc_t rb = make_rsrc(bt + (size_t)n0 * K2, rsrc_bytes(bt + (size_t)n0 * K2, bt + (size_t)N * K2));
  const rsrc_t rsa = make_rsrc(a_sc + (size_t)m0 * nsc,
                               rsrc_bytes(a_sc + (size_t)m0 * nsc, a_sc + (size_t)M * nsc));
  const rsrc_t rsb = make_rsrc(b_sc + (size_t)n0 * nsc,
                               rsrc_bytes(b_sc + (size_t)n0 * nsc, b_sc + (size_t)N * nsc));
  uint32_t voff[CH];
  int soff[CH];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = tid + 256 * i;
    const int r = c / (BK / 16), c16 = c % (BK / 16);
    voff[i] = (uint32_t)(r * K2 + c16 * 16);
    soff[i] = r * P + c16 * 16;
  }
  // scale dwords of this lane's rows: A rows wm*128 + mb*32 + l32, W^T rows wn*128 + nb*32 + l32
  uint32_t sa_off[4], sb_off[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) sa_off[mb] = (uint32_t)((wm * 128 + mb * 32 + l32) * nsc);
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) sb_off[nb] = (uint32_t)((wn * 128 + nb * 32 + l32) * nsc);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  u32x4 pa[CH], pb[CH];
  auto load_piece = [&](int i, int kt) {    // K steps past the end re-read the last one
    kt = min(kt, nkt - 1);
    const uint32_t kb = (uint32_t)(kt * BK);
    pa[i] = buf_ld16(ra, voff[i], kb);
    pb[i] = buf_ld16(rb, voff[i], kb);
  };
  auto store_piece = [&](int i, int buf) {
    st16(As(buf) + soff[i], pa[i]);
    st16(Bs(buf) + soff[i], pb[i]);
  };
  uint32_t sa[4], sb[4], sa_n[4], sb_n[4];
  auto load_scales = [&](uint32_t* da, uint32_t* db, int kt) {
    kt = min(kt, nkt - 1);
    const int kb = kt * 4;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      da[mb] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsa, (int)sa_off[mb], kb, 0);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      db[nb] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsb, (int)sb_off[nb], kb, 0);
  };
#pragma unroll
  for (int i = 0; i < CH; ++i) load_piece(i, 0);
#pragma unroll
  for (int i = 0; i < CH; ++i) store_piece(i, 0);
#pragma unroll
  for (int i = 0; i < CH; ++i) load_piece(i, 1);
  load_scales(sa, sb, 0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    load_scales(sa_n, sb_n, kt + 1);
    const uint8_t* Ab = As(kt & 1) + (wm * 128 + l32) * P + hg * 16;
    const uint8_t* Bb = Bs(kt & 1) + (wn * 128 + l32) * P + hg * 16;
    uint32_t ssa[4], ssb[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) ssa[mb] = sa[mb] >> (8 * hg);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) ssb[nb] = sb[nb] >> (8 * hg);
    auto frag = [&](const uint8_t* base, int ks) {
      const u32x4 lo = ld16(base + ks * 64);
      const u32x4 hi = ld16(base + ks * 64 + 32);
      i32x8 f;
      f[0] = (int)lo[0]; f[1] = (int)lo[1]; f[2] = (int)lo[2]; f[3] = (int)lo[3];
      f[4] = (int)hi[0]; f[5] = (int)hi[1]; f[6] = (int)hi[2]; f[7] = (int)hi[3];
      return f;
    };
    i32x8 fm[2][4], fn[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fm[0][i] = frag(Ab + i * 32 * P, 0);
      fn[0][i] = frag(Bb + i * 32 * P, 0);
    }
#pragma unroll
    for (int ks = 0; ks < NSUB; ++ks) {
      const int cur = ks & 1, nxt = cur ^ 1;
      if (ks + 1 < NSUB) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fm[nxt][i] = frag(Ab + i * 32 * P, ks + 1);
          fn[nxt][i] = frag(Bb + i * 32 * P, ks + 1);
        }
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          if (ks == 0)
            acc[nb][mb] = mfma_mx<0>(fn[cur][nb], fm[cur][mb], acc[nb][mb], (int)ssb[nb], (int)ssa[mb]);
          else
            acc[nb][mb] = mfma_mx<2>(fn[cur][nb], fm[cur][mb], acc[nb][mb], (int)ssb[nb], (int)ssa[mb]);
        }
      // stage chunks of the next K step, request them for the one after
#pragma unroll
      for (int q = ks * CPS; q < (ks + 1) * CPS; ++q) {
        store_piece(q, (kt + 1) & 1);
        load_piece(q, kt + 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) sa[mb] = sa_n[mb];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) sb[nb] = sb_n[nb];
    lds_barrier();
  }
  // Epilogue: the 256 x 256 bf16 tile goes through LDS (the operand buffers
  // are free after the K loop) and leaves as 512-byte row segments, 16 bytes
  // per lane, instead of 8 bytes into each of 32 rows D * 2 bytes apart.
  constexpr int TP = BN + 8;   // tile pitch (bf16)
  static_assert(BM * TP * 2 <= 2 * (BM + BN) * P, "output tile fits in the operand buffers");
  bf16_t* tile = reinterpret_cast<bf16_t*>(&lds[0][0]);
  __syncthreads();             // every wave is done with the operand tiles
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        u32x2 pk;
        pk[0] = pack_bf16x2(acc[nb][mb][i4 * 4 + 0], acc[nb][mb][i4 * 4 + 1]);
        pk[1] = pack_bf16x2(acc[nb][mb][i4 * 4 + 2], acc[nb][mb][i4 * 4 + 3]);
        *reinterpret_cast<u32x2*>(&tile[(wm * 128 + mb * 32 + l32) * TP + wn * 128 + nb * 32 + 8 * i4 + 4 * hg]) = pk;
      }
  __syncthreads();
  const int c8 = (tid % (BN / 8)) * 8;
  const bool col_ok = n0 + c8 < N;   // N % 8 == 0
#pragma unroll 2
  for (int it = 0; it < BM * (BN / 8) / 256; ++it) {
    const int r = it * (256 / (BN / 8)) + tid / (BN / 8);
    const long long m = m0 + r;
    const u32x4 v = ld16(&tile[r * TP + c8]);
    if (m < M && col_ok) st16(out + (size_t)m * N + n0 + c8, v);
  }
}

hipError_t launch_merge_gemm_mx(const uint8_t* a, const uint8_t* a_sc, const uint8_t* bt,
                                const uint8_t* b_sc, uint16_t* out, long long M, int K2, int Dm,
                                hipStream_t s) {
  if (M == 0 || Dm == 0) return hipSuccess;
  if (K2 % kMxBK || Dm % 8) return hipErrorInvalidValue;
  const int tm = (int)((M + kMxBM - 1) / kMxBM), tn = (Dm + kMxBN - 1) / kMxBN;
  const int rpx = (tm + kNumXcd - 1) / kNumXcd;
  const int groups = (rpx + kMxGroupRows - 1) / kMxGroupRows;
  const long long grid = (long long)kNumXcd * groups * kMxGroupRows * tn;
  merge_gemm_mx_kernel<<<(unsigned)grid, 256, 0, s>>>(a, a_sc, bt, b_sc, out, M, K2, Dm, tm, tn, rpx);
  return hipGetLastError();
}

}  // namespace vdn
