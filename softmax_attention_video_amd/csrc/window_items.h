// Work items of the window + anchor Softmax kernels (forward and backward).
//
// Paper ("Video DeltaNet: A Video-Native Hybrid Attention for Livestream
// Video Generation"), method, local Softmax window: the non-anchor frames of
// one chunk share one key set -- at most three contiguous token spans
// (anchor 0, the window, anchor F-1) -- and an anchor frame's keys are the
// whole sequence.  The visibility relation is symmetric (a frame sees
// another exactly when that one sees it), so the same items also describe,
// for a group of key frames, the query spans that see them.
#pragma once

#include "vdn_common.h"
#include "vdn_internal.h"

namespace vdn {

// Row order of a 32-row MFMA A operand such that, in the 32 x 32 result,
// lane half g holds rows 16 g .. 16 g + 15 in register order: loading row
// key_perm(l % 32) into lane l makes register i of half g row 16 g + i.
__device__ __forceinline__ int key_perm(int m) { return ((m >> 2) & 1) * 16 + (m >> 3) * 4 + (m & 3); }

struct Item {
  int bh;            // b * H + h
  int q_begin, q_end;
  int nspan;
  int kb0, ke0, kb1, ke1, kb2, ke2, kb3, ke3;   // up to four key spans [kb, ke)
};

// Key tiles of BK over the (up to NS <= 4) spans, flattened: tile j of the
// walk starts at key ks and holds nk valid keys.  The lookup is plain
// arithmetic on the span index (no selects of struct members), which keeps
// the walk in scalar registers instead of private memory.
template <int BK, int NS>
struct SpanWalk {
  int n0, n01, n012, n;   // cumulative tile counts
  int o0, o1, o2, o3;     // key start of tile j in span i is j * BK + o_i
  int e0, e1, e2, e3;     // span ends
  __device__ __forceinline__ SpanWalk(const Item& it) {
    const int kb1 = it.nspan > 1 ? it.kb1 : 0, ke1 = it.nspan > 1 ? it.ke1 : 0;
    const int kb2 = it.nspan > 2 ? it.kb2 : 0, ke2 = it.nspan > 2 ? it.ke2 : 0;
    const int kb3 = NS > 3 && it.nspan > 3 ? it.kb3 : 0, ke3 = NS > 3 && it.nspan > 3 ? it.ke3 : 0;
    n0 = (it.ke0 - it.kb0 + BK - 1) / BK;
    n01 = n0 + (ke1 - kb1 + BK - 1) / BK;
    n012 = n01 + (ke2 - kb2 + BK - 1) / BK;
    n = n012 + (ke3 - kb3 + BK - 1) / BK;
    o0 = it.kb0;
    o1 = kb1 - n0 * BK;
    o2 = kb2 - n01 * BK;
    o3 = kb3 - n012 * BK;
    e0 = it.ke0; e1 = ke1; e2 = ke2; e3 = ke3;
  }
  __device__ __forceinline__ void tile(int j, int& ks, int& nk) const {
    const int s1 = j >= n0, s2 = j >= n01, s3 = NS > 3 && j >= n012;
    ks = j * BK + o0 + (o1 - o0) * s1 + (o2 - o1) * s2 + (o3 - o2) * s3;
    const int e = e0 + (e1 - e0) * s1 + (e2 - e1) * s2 + (e3 - e2) * s3;
    nk = min(BK, e - ks);
  }
};

// Appends the text span [L, L + nt) after the item's video spans.
__host__ __device__ inline void add_text_span(const Geometry& g, int nt, Item& it) {
  it.kb3 = it.ke3 = 0;
  if (nt <= 0) return;
  const int tb = (int)g.L, te = (int)(g.L + nt);
  if (it.nspan == 1) {
    it.kb1 = tb; it.ke1 = te;
  } else if (it.nspan == 2) {
    it.kb2 = tb; it.ke2 = te;
  } else {
    it.kb3 = tb; it.ke3 = te;
  }
  ++it.nspan;
}

// Frame roles of one chunk group, in frames: the non-anchor query frames
// [f0, f1) of chunk c and their key frames, at most three contiguous frame
// spans in ascending order -- [anchor 0] window [anchor F-1].  The window is
// the chunks c - wc .. c + wc clipped to the clip; an anchor frame is a
// separate span only when it lies outside the window.  Returns false when
// the chunk has no non-anchor frame.  This is the one definition of the
// visibility rule: the Softmax kernels decode their work items through it
// and the host-side plan (vdn_window_plan) builds its frame mask from it.
struct ChunkRoles {
  int f0, f1;
  int nspan;
  int b0, e0, b1, e1, b2, e2;
};
__host__ __device__ inline bool chunk_roles(int F, int cf, int wc, int anchors, int c,
                                            ChunkRoles& r) {
  int f0 = c * cf, f1 = (c + 1) * cf;
  if (f1 > F) f1 = F;
  if (anchors) {
    if (f0 == 0) f0 = 1;
    if (f1 == F) f1 = F - 1;
  }
  r.f0 = f0;
  r.f1 = f1;
  int lo = c - wc;
  lo = (lo < 0 ? 0 : lo) * cf;
  int hi = (c + wc + 1) * cf;
  hi = hi > F ? F : hi;
  const bool a_lo = anchors && lo > 0, a_hi = anchors && hi < F;
  r.b0 = a_lo ? 0 : lo;
  r.e0 = a_lo ? 1 : hi;
  r.b1 = a_lo ? lo : F - 1;
  r.e1 = a_lo ? hi : F;
  r.b2 = F - 1;
  r.e2 = F;
  r.nspan = 1 + (a_lo ? 1 : 0) + (a_hi ? 1 : 0);
  return f1 > f0;
}

// Work split of the window Softmax over query groups.  An "anchor group" is
// one anchor frame of one head (its keys: the whole clip); a "chunk group"
// the non-anchor frames of one chunk of one head.  Groups are cut into
// query tiles of bq rows.  MI355X deals workgroups round-robin to its 8
// XCDs (workgroup b runs on XCD b % 8), so each XCD gets a contiguous slice
// of the groups -- anchor groups first -- and the grid is 8 x the longest
// slice.
inline SoftmaxWork window_work(const Geometry& g, int bq) {
  SoftmaxWork w{};
  w.GA = g.anchors ? 2 * g.B * g.H : 0;
  w.GC = g.B * g.H * g.C;
  w.tA = (g.N + bq - 1) / bq;
  w.tC = (g.cf * g.N + bq - 1) / bq;
  w.pa = (w.GA + kNumXcd - 1) / kNumXcd;
  w.pc = (w.GC + kNumXcd - 1) / kNumXcd;
  int mx = 0;
  for (int x = 0; x < kNumXcd; ++x) {
    int na = w.GA - x * w.pa;
    na = na < 0 ? 0 : (na > w.pa ? w.pa : na);
    int nc = w.GC - x * w.pc;
    nc = nc < 0 ? 0 : (nc > w.pc ? w.pc : nc);
    int items = na * w.tA + nc * w.tC;
    mx = items > mx ? items : mx;
  }
  w.grid = mx * kNumXcd;
  return w;
}

// Decode workgroup id -> (query range, key spans).  Returns false if idle.
// TEXT: append a span of the first nt text keys (none if nt == 0).
template <bool TEXT>
__host__ __device__ inline bool decode_item(const Geometry& g, const SoftmaxWork& w, int bq,
                                            int bid, int nt, Item& it, int& q0) {
  const int x = bid % kNumXcd;
  int k = bid / kNumXcd;
  const int a0 = x * w.pa;
  int na = w.GA - a0;
  na = na < 0 ? 0 : (na > w.pa ? w.pa : na);
  const long long N = g.N;
  if (k < na * w.tA) {
    const int ga = a0 + k / w.tA;
    const int tile = k % w.tA;
    it.bh = ga >> 1;
    const int f = (ga & 1) ? g.F - 1 : 0;
    it.q_begin = (int)(f * N);
    it.q_end = (int)((f + 1) * N);
    it.nspan = 1;
    it.kb0 = 0;
    it.ke0 = (int)g.L;
    it.kb1 = it.ke1 = it.kb2 = it.ke2 = it.kb3 = it.ke3 = 0;
    if (TEXT) add_text_span(g, nt, it);
    q0 = it.q_begin + tile * bq;
    return true;
  }
  k -= na * w.tA;
  const int gc = x * w.pc + k / w.tC;
  const int tile = k % w.tC;
  if (gc >= w.GC || gc >= (x + 1) * w.pc) return false;
  it.bh = gc / g.C;
  ChunkRoles r;
  if (!chunk_roles(g.F, g.cf, g.wc, g.anchors, gc % g.C, r)) return false;
  const int nN = (int)N;
  it.q_begin = r.f0 * nN;
  it.q_end = r.f1 * nN;
  it.kb0 = r.b0 * nN;
  it.ke0 = r.e0 * nN;
  it.kb1 = r.b1 * nN;
  it.ke1 = r.e1 * nN;
  it.kb2 = r.b2 * nN;
  it.ke2 = r.e2 * nN;
  it.nspan = r.nspan;
  it.kb3 = it.ke3 = 0;
  if (TEXT) add_text_span(g, nt, it);
  q0 = it.q_begin + tile * bq;
  return q0 < it.q_end;
}

}  // namespace vdn
