// Window + boundary-anchor Softmax branch of VDN attention.
//
// Paper ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream
// Video Generation"), method, local Softmax window: a query chunk of
// chunk_frames latent frames sees itself and window_chunks chunks on each
// side; with anchors every frame also sees frames 0 and F-1 and those two
// frames see every frame; each key frame counts once.
//
// Optionally (method, bidirectional linear attention: the prompt stays
// directly visible to the Softmax branch) the Ts text tokens are keys of
// every video query as well, in the same softmax.
//
// Work decomposition.  All non-anchor query frames of one chunk share one
// key set, so a "chunk group" is the contiguous query range of a chunk minus
// its anchor frames, and its keys are at most three contiguous token spans
// (anchor 0, the window, anchor F-1).  An "anchor group" is one anchor frame,
// whose keys are the whole sequence.  The text keys are one more span, after
// the video ones, numbered L .. L+Ts-1 in the walk.  Groups are cut into
// query tiles; one workgroup owns one tile and streams the key spans through
// LDS with an online softmax (no mask tensor, no gathered copies).
//
// XCD-aware order: MI355X deals workgroups round-robin to its 8 XCDs, so
// blockIdx b runs on XCD b % 8.  Each XCD gets a contiguous slice of groups
// (consecutive chunks of the same head share 2/3 of their key windows in
// that XCD's L2), anchor groups (7x longer at 120 frames) first.
#include "vdn_common.h"
#include "vdn_internal.h"
#include "window_items.h"

#include <math.h>

#include <type_traits>

namespace vdn {

// -------------------------------------------------------------------------
// bf16 MFMA flash kernel.  512 threads = 8 waves of 32 queries each (256
// queries per workgroup), two waves per SIMD.  The kernel is compiled with
// MFMA results in arch VGPRs (not AGPRs) so the softmax reads S without
// accumulator-register moves.
//   S^T (keys x queries) = K Q^T  on v_mfma_f32_32x32x16_bf16;
//   O^T (dv x queries)  += V^T P^T, with V pre-transposed to [D, L].
// In the S^T accumulator a lane holds one query (lane % 32) and 16 keys.  K
// rows are loaded in a permuted order so that lane half g holds keys
// 16g..16g+15 of each 32-key block in register order; those registers then
// feed the PV product directly as its B operand, matching 16 contiguous
// bytes of V^T.
//
// Software pipeline per 32-key block b: the QK^T MFMAs of block b+1 are
// issued while the VALU turns S_b into P_b, then PV of block b.  Key tiles
// (96 keys at D = 128, 128 at D = 64) are staged global -> registers -> LDS
// one piece per block, with one workgroup barrier per tile.
//
// Online softmax with a lazy reference: O and l are kept relative to a
// running reference m; P is computed against it and the reference only
// moves (rescaling O and l, recomputing P) when a lane's partial row sum of
// the block exceeds kLazySum, which bounds every probability it holds.  No
// per-block row max is needed on the common path.  This is exact: the final
// O / l does not depend on the reference.
// -------------------------------------------------------------------------
struct WinArgs {
  Geometry g;
  SoftmaxWork w;
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* kt;      // text keys [B,H,Ts,D]
  const bf16_t* vt;      // V^T [B,H,D,Lp]: video keys, then text keys
  long long vt_pitch;    // Lp
  const float* g_s;
  bf16_t* out;
  float* lse;
  float scale_log2;
};

constexpr int kWinNW = 8;                  // waves per workgroup, 32 queries each
constexpr int kWinBQ = kWinNW * 32;        // queries per workgroup
static_assert(kWinBQ == kWinMfmaBQ, "query rows per workgroup");
constexpr float kLazySum = 256.f;


template <int D, bool TEXT>
__global__ __launch_bounds__(kWinNW * 64) void window_softmax_mfma_kernel(WinArgs a) {
  // 96-key tiles at D = 128 keep two K and three V buffers within LDS.
  constexpr int BQ = kWinBQ, BK = D == 128 ? 96 : 128, NT = kWinNW * 64;
  constexpr int KP = D + 8;    // padded pitches (bf16 elements) against bank conflicts
  constexpr int VP = BK + 8;
  constexpr int NKK = D / 16;  // k-steps of QK^T
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  constexpr int NB = BK / 32;  // 32-key blocks per tile
  constexpr int KCH = BK * D / 8 / NT;   // 16-byte chunks per thread per tile
  constexpr int VCH = D * BK / 8 / NT;
  static_assert(KCH * NT * 8 == BK * D && VCH * NT * 8 == D * BK, "tile split");
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][BK * KP];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[3][D * VP];

  const Geometry& g = a.g;
  Item it;
  int q0;
  // The walk holds the text keys in whole 16-key groups; the last Ts % 16
  // are one masked block after it.
  const int t16 = TEXT ? g.Ts & ~15 : 0;
  if (!decode_item<TEXT>(g, a.w, BQ, blockIdx.x, t16, it, q0)) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63, hg = lane >> 5, l32 = lane & 31;
  const long long L = g.L;
  const long long Lp = a.vt_pitch;
  const bf16_t* Q = a.q + (size_t)it.bh * L * D;
  const bf16_t* K = a.k + (size_t)it.bh * L * D;
  const bf16_t* Kt = a.kt + (size_t)it.bh * g.Ts * D;
  const bf16_t* Vt = a.vt + (size_t)it.bh * Lp * D;
  const float sl2 = a.scale_log2;

  bf16x8 qf[NKK];
  {
    const int qrow = q0 + wave * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 v = {0, 0, 0, 0};
      if (qrow < it.q_end) v = ld16(Q + (size_t)qrow * D + kk * 16 + hg * 8);
      qf[kk] = as_bf16x8(v);
    }
  }
  f32x16 o[NDB];
#pragma unroll
  for (int b = 0; b < NDB; ++b) o[b] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int krow_perm = key_perm(l32);
  const SpanWalk<BK, TEXT ? 4 : 3> walk(it);

  // Tile staging.  A tile is KCH K chunks and VCH V^T chunks of 16 bytes
  // per thread, cut into NB pieces; one piece is stored to LDS and the same
  // piece of the tile two ahead is requested per 32-key block, so the
  // workgroup's vector-memory requests are spread over the tile instead of
  // arriving in one burst.  Loads are raw buffer loads: per-lane byte offsets
  // are loop invariant, the tile position goes into the descriptor base; K
  // rows past the tile's valid keys fall outside the descriptor and read as
  // zero, V^T columns past them are steered out of range the same way.
  // Text tiles (keys L and up) take their K rows from the text keys.
  constexpr int CH = KCH + VCH, CPP = CH / NB;
  static_assert(CPP * NB == CH, "pieces");
  u32x4 cA[CH], cB[CH];   // staging registers of even / odd tiles
  const uint32_t vt_bytes = (uint32_t)min((long long)D * Lp * 2, 0x7FFFFFF0ll);
  const int Li = (int)L;
  auto load_keys = [&](u32x4* creg, int p, int ks, int nk) {
    const bf16_t* kbase = !TEXT || ks < Li ? K + (size_t)ks * D : Kt + (size_t)(ks - Li) * D;
    const rsrc_t krs = make_rsrc(kbase, (uint32_t)nk * D * 2);
    const rsrc_t vrs = make_rsrc(Vt + ks, vt_bytes - (uint32_t)ks * 2);
#pragma unroll
    for (int q = p * CPP; q < (p + 1) * CPP; ++q) {
      if (q < KCH) {
        const int c = tid + NT * q;
        creg[q] = buf_ld16(krs, (uint32_t)((c / (D / 8)) * D + (c % (D / 8)) * 8) * 2);
      } else {
        const int c = tid + NT * (q - KCH);
        const int r = c / (BK / 8), c8 = c % (BK / 8);
        const uint32_t off = (uint32_t)(r * Lp + c8 * 8) * 2;
        creg[q] = buf_ld16(vrs, c8 * 8 < nk ? off : 0x80000000u);
      }
    }
  };
  auto load_piece = [&](u32x4* creg, int p, int j) {   // tiles past the walk read as zeros
    int ks, nk;
    walk.tile(j, ks, nk);
    if (j >= walk.n) ks = 0, nk = 0;
    load_keys(creg, p, ks, nk);
  };
  auto store_piece = [&](const u32x4* creg, int p, int j) {
#pragma unroll
    for (int q = p * CPP; q < (p + 1) * CPP; ++q) {
      if (q < KCH) {
        const int c = tid + NT * q;
        st16(&Ks[j & 1][(c / (D / 8)) * KP + (c % (D / 8)) * 8], creg[q]);
      } else {
        const int c = tid + NT * (q - KCH);
        st16(&Vs[j % 3][(c / (BK / 8)) * VP + (c % (BK / 8)) * 8], creg[q]);
      }
    }
  };
  // S^T of one 32-key block: lane half hg holds keys 16 hg .. 16 hg + 15.
  auto qk = [&](const bf16_t* Kb, int blk) {
    f32x16 s = {};
    const bf16_t* krow = Kb + (blk * 32 + krow_perm) * KP + hg * 8;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) s = mfma32x32x16(as_bf16x8(ld16(krow + kk * 16)), qf[kk], s);
    return s;
  };
  // P of one block relative to the running reference m_run.  The lane's
  // partial row sum bounds every p it holds, so while it stays <= 2^8 no p
  // can overflow and the reference may stay.  Otherwise (also on the first
  // block, where m_run = -inf makes every p infinite) the block max moves the
  // reference, O and l are rescaled, and P is recomputed.  nv is the number
  // of valid keys in the block (0..32, workgroup-uniform); a lane half with
  // none is masked through nm.  With MASK (only the block of the last
  // Ts % 16 text keys) a half may hold some: its missing keys get offset
  // -inf.
  auto probs = [&](auto mask, const f32x16& s, int nv, bf16x8* pb) {
    constexpr bool MASK = decltype(mask)::value;
    const int nvh = nv - hg * 16;
    const bool valid = nvh > 0;
    // offset of key i: nm on valid keys, -inf on masked ones
    auto key_nm = [&](int i, float nm) { return !MASK || i < nvh ? nm : -INFINITY; };
    float ls = 0.f;
    {
      const float nm = valid ? -m_run : -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[i], sl2, key_nm(i, nm)));
        ls += p;
        pb[i >> 3][i & 7] = static_cast<__bf16>(p);
      }
    }
    // Issue order for the scheduler: the next block's K fragment reads, then
    // its QK^T MFMAs spread one per six VALU instructions of this block's
    // exponentials, so the matrix core and the VALU of a wave overlap.
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // 8 LDS reads
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0); // 1 MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0); // 6 VALU
    }
    if (__any(!(ls <= kLazySum))) {
      float m = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) m = fmaxf(m, !MASK || i < nvh ? s[i] : -INFINITY);
      m = valid ? m : -INFINITY;
      const float m_new = fmaxf(m_run, half_max(m) * sl2);
      const float corr = m_new == m_run ? 1.f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= corr;
#pragma unroll
      for (int b = 0; b < NDB; ++b) o[b] *= corr;
      const float nm = valid ? -m_run : -INFINITY;
      ls = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p = fast_exp2(fmaf(s[i], sl2, key_nm(i, nm)));
        ls += p;
        pb[i >> 3][i & 7] = static_cast<__bf16>(p);
      }
    }
    l_run += ls;
  };

#pragma unroll
  for (int p = 0; p < NB; ++p) load_piece(cA, p, 0);
#pragma unroll
  for (int p = 0; p < NB; ++p) store_piece(cA, p, 0);
#pragma unroll
  for (int p = 0; p < NB; ++p) load_piece(cB, p, 1);
  store_piece(cB, 0, 1);
#pragma unroll
  for (int p = 0; p < NB; ++p) load_piece(cA, p, 2);
  load_piece(cB, 0, 3);
  __syncthreads();
  int ks, nk;
  walk.tile(0, ks, nk);
  f32x16 s_cur = qk(Ks[0], 0);
  int nv_cur = min(nk, 32);
  // Pieces are requested two tiles ahead of their LDS store, in the register
  // set of the tile's parity.
  constexpr std::integral_constant<bool, false> kNoMask{};
  auto tile_body = [&](int j, u32x4* c_near, u32x4* c_far) {
    const bf16_t* Kb = Ks[j & 1];
    const bf16_t* Vb = Vs[j % 3];
    const bf16_t* Kn = Ks[(j + 1) & 1];
    int ks1 = 0, nk1 = 0;
    if (j + 1 < walk.n) walk.tile(j + 1, ks1, nk1);
#pragma unroll
    for (int kb2 = 0; kb2 < NB; ++kb2) {
      // (1) S of the next block on the matrix core, P of this block on the VALU
      const f32x16 s_next = kb2 + 1 < NB ? qk(Kb, kb2 + 1) : qk(Kn, 0);
      const int nv_next = kb2 + 1 < NB ? max(0, min(nk - (kb2 + 1) * 32, 32)) : min(nk1, 32);
      bf16x8 pb[2];
      probs(kNoMask, s_cur, nv_cur, pb);
      // (2) O += V P of this block
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int b = 0; b < NDB; ++b) {
          const bf16x8 vf = as_bf16x8(ld16(Vb + (b * 32 + l32) * VP + kb2 * 32 + hg * 16 + h2 * 8));
          o[b] = mfma32x32x16(vf, pb[h2], o[b]);
        }
      s_cur = s_next;
      nv_cur = nv_next;
      // Stage piece p of the next tile (of the one after, on the last
      // block); one barrier per tile, once the next tile is complete.  K
      // tiles are read one block ahead of V tiles, so K needs two buffers
      // and V three.  Stores and loads are unconditional (tiles past the
      // walk are zeros), which keeps the vector-memory wait counts exact.
      {
        const int p = (kb2 + 1) % NB;
        const bool far = kb2 == NB - 1;
        const int st = j + 1 + (far ? 1 : 0);
        u32x4* c = far ? c_far : c_near;
        store_piece(c, p, st);
        if (kb2 == NB - 2) lds_barrier();
        load_piece(c, p, st + 2);
      }
    }
    nk = nk1;
  };
  for (int j = 0; j < walk.n; j += 2) {
    tile_body(j, cB, cA);
    if (j + 1 < walk.n) tile_body(j + 1, cA, cB);
  }
  if constexpr (TEXT) {
    // the last Ts % 16 text keys: one 32-key block with a per-key mask
    const int rem = g.Ts - t16;
    if (rem > 0) {
      __syncthreads();   // every wave is done with the walk's LDS tiles
#pragma unroll
      for (int p = 0; p < NB; ++p) load_keys(cA, p, Li + t16, rem);
#pragma unroll
      for (int p = 0; p < NB; ++p) store_piece(cA, p, 0);
      __syncthreads();
      bf16x8 pb[2];
      probs(std::integral_constant<bool, true>{}, qk(Ks[0], 0), rem, pb);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int b = 0; b < NDB; ++b) {
          const bf16x8 vf = as_bf16x8(ld16(Vs[0] + (b * 32 + l32) * VP + hg * 16 + h2 * 8));
          o[b] = mfma32x32x16(vf, pb[h2], o[b]);
        }
    }
  }

  const int bidx = it.bh / g.H, h = it.bh % g.H;
  const float l_tot = half_sum(l_run);
  const int qrow = q0 + wave * 32 + l32;
  if (qrow < it.q_end) {
    const float gate = a.g_s ? a.g_s[(size_t)it.bh * L + qrow] : 1.f;
    const float sc = gate / l_tot;
    bf16_t* orow = a.out + (((size_t)bidx * L + qrow) * g.H + h) * D;
#pragma unroll
    for (int b = 0; b < NDB; ++b)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int dv = b * 32 + 8 * i4 + 4 * hg;
        u32x2 pk;
        pk[0] = pack_bf16x2(o[b][i4 * 4 + 0] * sc, o[b][i4 * 4 + 1] * sc);
        pk[1] = pack_bf16x2(o[b][i4 * 4 + 2] * sc, o[b][i4 * 4 + 3] * sc);
        *reinterpret_cast<u32x2*>(orow + dv) = pk;
      }
    if (a.lse && hg == 0) a.lse[(size_t)it.bh * L + qrow] = m_run * kLn2 + logf(l_tot);
  }
}

bool window_softmax_mfma_ok(const Geometry& g) {
  // whole 16-key groups in every video span; V^T of one head addressed by a
  // single 32-bit buffer descriptor
  return (g.D == 64 || g.D == 128) && (g.N % 16 == 0) &&
         (long long)g.D * softmax_vt_pitch(g) * 2 <= 0x7FFFFFF0ll;
}

hipError_t launch_window_softmax_mfma(const Geometry& g, const uint16_t* q, const uint16_t* k,
                                      const uint16_t* k_text, const uint16_t* vt,
                                      const float* g_s, uint16_t* out, float* lse, float scale,
                                      hipStream_t s) {
  if (g.Ts > 0 && !k_text) return hipErrorInvalidValue;
  WinArgs a;
  a.g = g;
  a.w = window_work(g, kWinBQ);
  a.q = q; a.k = k; a.kt = k_text; a.vt = vt; a.g_s = g_s; a.out = out; a.lse = lse;
  a.vt_pitch = softmax_vt_pitch(g);
  a.scale_log2 = scale * kLog2e;
  if (a.w.grid == 0) return hipSuccess;
  if (g.D == 128 && g.Ts > 0)
    window_softmax_mfma_kernel<128, true><<<a.w.grid, kWinNW * 64, 0, s>>>(a);
  else if (g.D == 128)
    window_softmax_mfma_kernel<128, false><<<a.w.grid, kWinNW * 64, 0, s>>>(a);
  else if (g.Ts > 0)
    window_softmax_mfma_kernel<64, true><<<a.w.grid, kWinNW * 64, 0, s>>>(a);
  else
    window_softmax_mfma_kernel<64, false><<<a.w.grid, kWinNW * 64, 0, s>>>(a);
  return hipGetLastError();
}

// -------------------------------------------------------------------------
// [rows, cols] -> [cols, rows] per batch, bf16, through a 64x64 LDS tile.
// Used to lay V (and the text values) out key-contiguous for the PV product
// and the output projections out K-contiguous for the merge.  Source rows
// src_rows .. rows-1 read as zeros (the padding of the text columns).
// -------------------------------------------------------------------------
struct TransposeArgs {
  const bf16_t* src;
  bf16_t* dst;
  long long rows, src_rows;
  int cols;
  long long ldd, dst_bstride;
};

__global__ __launch_bounds__(256) void transpose_bf16_kernel(TransposeArgs a) {
  __shared__ bf16_t t[64][65];
  const long long r0 = (long long)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const bf16_t* src = a.src + (size_t)blockIdx.z * a.src_rows * a.cols;
  bf16_t* dst = a.dst + (size_t)blockIdx.z * a.dst_bstride;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < 64; r += 4) {
    const long long gr = r0 + r;
    const int gc = c0 + tx;
    t[r][tx] = (gr < a.src_rows && gc < a.cols) ? src[gr * a.cols + gc] : (bf16_t)0;
  }
  __syncthreads();
  for (int c = ty; c < 64; c += 4) {
    const int gc = c0 + c;
    const long long gr = r0 + tx;
    if (gc < a.cols && gr < a.rows) dst[(size_t)gc * a.ldd + gr] = t[tx][c];
  }
}

// Same transpose with 16-byte global accesses (rows, cols, ldd multiples of
// 8 and a 16-byte aligned destination).
__global__ __launch_bounds__(256) void transpose16_bf16_kernel(TransposeArgs a) {
  __shared__ bf16_t t[64][66];
  const long long r0 = (long long)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const bf16_t* src = a.src + (size_t)blockIdx.z * a.src_rows * a.cols;
  bf16_t* dst = a.dst + (size_t)blockIdx.z * a.dst_bstride;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ch = threadIdx.x + 256 * i;
    const int r = ch >> 3, c8 = (ch & 7) * 8;
    u32x4 v = {0, 0, 0, 0};
    if (r0 + r < a.src_rows && c0 + c8 < a.cols) v = ld16(src + (size_t)(r0 + r) * a.cols + c0 + c8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      t[r][c8 + 2 * j] = (bf16_t)(v[j] & 0xFFFFu);
      t[r][c8 + 2 * j + 1] = (bf16_t)(v[j] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ch = threadIdx.x + 256 * i;
    const int c = ch >> 3, r8 = (ch & 7) * 8;
    if (c0 + c >= a.cols || r0 + r8 >= a.rows) continue;
    u32x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      v[j] = (uint32_t)t[r8 + 2 * j][c] | ((uint32_t)t[r8 + 2 * j + 1][c] << 16);
    st16(dst + (size_t)(c0 + c) * a.ldd + r0 + r8, v);
  }
}

hipError_t launch_transpose_bf16(const uint16_t* src, uint16_t* dst, long long rows,
                                 long long src_rows, int cols, long long ldd,
                                 long long dst_bstride, long long batch, hipStream_t s) {
  if (rows == 0 || cols == 0 || batch == 0) return hipSuccess;
  if (src_rows > rows || ldd < rows) return hipErrorInvalidValue;
  if (src_rows > 0 && !src) return hipErrorInvalidValue;
  const TransposeArgs a{src, dst, rows, src_rows, cols, ldd, dst_bstride};
  dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((cols + 63) / 64), (unsigned)batch);
  if (rows % 8 == 0 && cols % 8 == 0 && ldd % 8 == 0 && dst_bstride % 8 == 0 &&
      ((uintptr_t)dst & 15) == 0 && ((uintptr_t)src & 15) == 0)
    transpose16_bf16_kernel<<<grid, 256, 0, s>>>(a);
  else
    transpose_bf16_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

// -------------------------------------------------------------------------
// Generic SIMT kernel (fp32 storage, any D <= 128, any N): one thread per
// query, keys staged through LDS 32 at a time, fp32 online softmax.
// -------------------------------------------------------------------------
template <typename T, int DMAX>
__global__ __launch_bounds__(128) void window_softmax_simt_kernel(Geometry g, SoftmaxWork w,
                                                                  const T* __restrict__ qp,
                                                                  const T* __restrict__ kp,
                                                                  const T* __restrict__ vp,
                                                                  const T* __restrict__ ktp,
                                                                  const T* __restrict__ vtp,
                                                                  const float* __restrict__ g_s,
                                                                  T* __restrict__ out,
                                                                  float* __restrict__ lse,
                                                                  float scale_log2) {
  constexpr int BQ = kWinSimtBQ, BK = 32;
  __shared__ float Ks[BK][DMAX + 1];
  __shared__ float Vs[BK][DMAX + 1];
  Item it;
  int q0;
  if (!decode_item<true>(g, w, BQ, blockIdx.x, g.Ts, it, q0)) return;
  const int D = g.D;
  const long long L = g.L;
  const int qrow = q0 + threadIdx.x;
  const bool qvalid = qrow < it.q_end;
  const size_t base = (size_t)it.bh * L * D;
  const size_t tbase = (size_t)it.bh * g.Ts * D;
  float qv[DMAX], ov[DMAX];
#pragma unroll
  for (int j = 0; j < DMAX; ++j) {
    qv[j] = (j < D && qvalid) ? Elem<T>::load(qp, base + (size_t)qrow * D + j) : 0.f;
    ov[j] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const SpanWalk<BK, 4> walk(it);
  for (int jt = 0; jt < walk.n; ++jt) {
    {
      int ks, nk;
      walk.tile(jt, ks, nk);
      // a tile lies in one span: video keys, or text keys (ks >= L)
      const bool text = ks >= L;
      const T* kb = text ? ktp + tbase + (size_t)(ks - L) * D : kp + base + (size_t)ks * D;
      const T* vb = text ? vtp + tbase + (size_t)(ks - L) * D : vp + base + (size_t)ks * D;
      __syncthreads();
      for (int e = threadIdx.x; e < BK * D; e += blockDim.x) {
        const int r = e / D, c = e % D;
        Ks[r][c] = r < nk ? Elem<T>::load(kb, (size_t)r * D + c) : 0.f;
        Vs[r][c] = r < nk ? Elem<T>::load(vb, (size_t)r * D + c) : 0.f;
      }
      __syncthreads();
      for (int r = 0; r < nk; ++r) {
        float dot = 0.f;
#pragma unroll
        for (int j = 0; j < DMAX; ++j)
          if (j < D) dot = fmaf(qv[j], Ks[r][j], dot);
        const float sv = dot * scale_log2;
        const float m_new = fmaxf(m_run, sv);
        const float corr = exp2f(m_run - m_new);
        const float p = exp2f(sv - m_new);
        l_run = l_run * corr + p;
#pragma unroll
        for (int j = 0; j < DMAX; ++j)
          if (j < D) ov[j] = ov[j] * corr + p * Vs[r][j];
        m_run = m_new;
      }
    }
  }
  if (!qvalid) return;
  const int bidx = it.bh / g.H, h = it.bh % g.H;
  const float gate = g_s ? g_s[(size_t)it.bh * L + qrow] : 1.f;
  const float sc = gate / l_run;
  const size_t ob = (((size_t)bidx * L + qrow) * g.H + h) * D;
#pragma unroll
  for (int j = 0; j < DMAX; ++j)
    if (j < D) Elem<T>::store(out, ob + j, ov[j] * sc);
  if (lse) lse[(size_t)it.bh * L + qrow] = m_run * kLn2 + logf(l_run);
}

template <typename T>
hipError_t launch_window_softmax_simt(const Geometry& g, const T* q, const T* k, const T* v,
                                      const T* k_text, const T* v_text, const float* g_s, T* out,
                                      float* lse, float scale, hipStream_t s) {
  if (g.Ts > 0 && (!k_text || !v_text)) return hipErrorInvalidValue;
  const SoftmaxWork w = window_work(g, kWinSimtBQ);
  if (w.grid == 0) return hipSuccess;
  const float sl2 = scale * kLog2e;
  if (g.D <= 16)
    window_softmax_simt_kernel<T, 16><<<w.grid, 128, 0, s>>>(g, w, q, k, v, k_text, v_text, g_s, out, lse, sl2);
  else if (g.D <= 32)
    window_softmax_simt_kernel<T, 32><<<w.grid, 128, 0, s>>>(g, w, q, k, v, k_text, v_text, g_s, out, lse, sl2);
  else if (g.D <= 64)
    window_softmax_simt_kernel<T, 64><<<w.grid, 128, 0, s>>>(g, w, q, k, v, k_text, v_text, g_s, out, lse, sl2);
  else
    window_softmax_simt_kernel<T, 128><<<w.grid, 128, 0, s>>>(g, w, q, k, v, k_text, v_text, g_s, out, lse, sl2);
  return hipGetLastError();
}

template hipError_t launch_window_softmax_simt<float>(const Geometry&, const float*, const float*,
                                                      const float*, const float*, const float*,
                                                      const float*, float*, float*, float,
                                                      hipStream_t);
template hipError_t launch_window_softmax_simt<bf16_t>(const Geometry&, const bf16_t*,
                                                       const bf16_t*, const bf16_t*, const bf16_t*,
                                                       const bf16_t*, const float*, bf16_t*, float*,
                                                       float, hipStream_t);

}  // namespace vdn
