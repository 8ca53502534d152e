// Block geometry of an LCSA problem, shared by the host layer and the kernels.
//
// Blocks are 2x8x8 tokens (t x h x w). Block-causal visibility follows FlashVSR's stage-2 causal
// masking (fmread summary, sec. 2.2): key block j is visible from query block i iff its temporal
// block (latent frame / 2) is not later than i's. The locality window of sec. 2.3 is applied per
// spatial axis at block granularity: w_b = win / 8 blocks (odd), r = (w_b - 1) / 2;
//   truncated:  [c - r, c + r] cut to [0, n)
//   preserving: a w_b-wide window slid inward at the frame edge, start = clamp(c - r, 0, n - w_b).
#pragma once

#include <math.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define LCSA_HD __host__ __device__ __forceinline__
#else
#define LCSA_HD inline
#endif

namespace lcsa {

constexpr int kBlkT = 2, kBlkH = 8, kBlkW = 8;
constexpr int kBlkTokens = kBlkT * kBlkH * kBlkW;  // 128

struct Geom {
  int32_t H, W;          // tokens per frame
  int32_t Hb, Wb;        // blocks per frame: ceil(H / 8), ceil(W / 8)
  int32_t bpt;           // blocks per temporal block = Hb * Wb
  int32_t nqb, nkb;      // query / key blocks per (batch, head)
  int32_t q_tb0;         // absolute temporal block of query block 0 (q_frame0 / 2)
  int32_t win_mode;      // 0 none, 1 / 2 block-granular truncated / preserving, 3 / 4 token-granular
  int32_t wbh, wbw;      // window width in blocks per axis (odd), modes 1 and 2
  int32_t wth, wtw;      // window width in tokens per axis, modes 3 and 4
};

constexpr int kWinTokenTruncated = 3, kWinTokenPreserving = 4;

LCSA_HD bool token_window(const Geom& g) { return g.win_mode >= kWinTokenTruncated; }

// Token-granular window along an axis of n tokens: the w tokens starting at c - (w - 1) / 2 (the
// query's own position is inside; an even w has one more token after c than before), cut to [0, n)
// (truncated) or shifted inside (preserving; the whole axis when n <= w). Inclusive [lo, hi]; lo and
// hi never decrease as c grows.
LCSA_HD void tok_range(bool preserve, int c, int n, int w, int* lo, int* hi) {
  int s = c - (w - 1) / 2;
  if (preserve) {
    if (n <= w) {
      *lo = 0;
      *hi = n - 1;
      return;
    }
    s = s < 0 ? 0 : (s > n - w ? n - w : s);
    *lo = s;
    *hi = s + w - 1;
  } else {
    const int e = s + w - 1;
    *lo = s < 0 ? 0 : s;
    *hi = e > n - 1 ? n - 1 : e;
  }
}

// Inclusive block range [lo, hi] visible along one axis of n blocks from block c.
LCSA_HD void win_range(int mode, int c, int n, int wb, int* lo, int* hi) {
  if (mode == 0 || wb >= 2 * n - 1) {
    *lo = 0;
    *hi = n - 1;
    return;
  }
  const int r = (wb - 1) / 2;
  if (mode == 1) {
    *lo = c - r < 0 ? 0 : c - r;
    *hi = c + r > n - 1 ? n - 1 : c + r;
  } else {
    if (n <= wb) {
      *lo = 0;
      *hi = n - 1;
      return;
    }
    int s = c - r;
    s = s < 0 ? 0 : s;
    s = s > n - wb ? n - wb : s;
    *lo = s;
    *hi = s + wb - 1;
  }
}

// Absolute temporal block, block row and block column of query block i.
LCSA_HD void qblock_coords(const Geom& g, int i, int* tb, int* hb, int* wb) {
  const int tr = i / g.bpt, rem = i - tr * g.bpt;
  *tb = g.q_tb0 + tr;
  *hb = rem / g.Wb;
  *wb = rem - (rem / g.Wb) * g.Wb;
}

// Rows (1..8) of block row hb and columns (1..8) of block column wb that lie inside the grid: blocks
// start at the spatial origin, so only the last block row and column can be partial.
LCSA_HD int block_rows(const Geom& g, int hb) {
  const int r = g.H - kBlkH * hb;
  return r < kBlkH ? r : kBlkH;
}
LCSA_HD int block_cols(const Geom& g, int wb) {
  const int c = g.W - kBlkW * wb;
  return c < kBlkW ? c : kBlkW;
}

// Visible spatial window of query block i: block rows [h0, h1], block columns [w0, w1];
// returns the last visible temporal block. With a token-granular window a key block is visible when
// some token of i sees some token of it: per axis, the union of the windows of i's tokens, which is
// [lo(first), hi(last)] since the bounds are monotone.
LCSA_HD void qblock_window_at(const Geom& g, int hb, int wb, int* h0, int* h1, int* w0, int* w1);

LCSA_HD int qblock_window(const Geom& g, int i, int* h0, int* h1, int* w0, int* w1) {
  int tb, hb, wb;
  qblock_coords(g, i, &tb, &hb, &wb);
  qblock_window_at(g, hb, wb, h0, h1, w0, w1);
  return tb;
}

// The window of query block (hb, wb) (any temporal block): inclusive key-block rows [h0, h1] and
// columns [w0, w1].
LCSA_HD void qblock_window_at(const Geom& g, int hb, int wb, int* h0, int* h1, int* w0, int* w1) {
  if (token_window(g)) {
    const bool pres = g.win_mode == kWinTokenPreserving;
    int lo, hi, lo2, hi2;
    tok_range(pres, 8 * hb, g.H, g.wth, &lo, &hi);
    tok_range(pres, 8 * hb + block_rows(g, hb) - 1, g.H, g.wth, &lo2, &hi2);
    *h0 = lo / 8;
    *h1 = hi2 / 8;
    tok_range(pres, 8 * wb, g.W, g.wtw, &lo, &hi);
    tok_range(pres, 8 * wb + block_cols(g, wb) - 1, g.W, g.wtw, &lo2, &hi2);
    *w0 = lo / 8;
    *w1 = hi2 / 8;
    return;
  }
  win_range(g.win_mode, hb, g.Hb, g.wbh, h0, h1);
  win_range(g.win_mode, wb, g.Wb, g.wbw, w0, w1);
}

// Unsigned division by a run-time constant d >= 1 as one multiply and a shift (Granlund-Montgomery
// round-up method): with l = ceil(log2 d), k = 32 + l and M = ceil(2^k / d), floor(n / d) equals
// floor(n * M / 2^k) for every n < 2^31 (M <= 2^33, so the product fits in 64 bits).
struct FastDiv {
  uint64_t m;
  uint32_t k;
  uint32_t d;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t p = uint64_t(1) << (32 + l);
  return FastDiv{(p + d - 1) / d, 32 + l, d};
}

LCSA_HD uint32_t fast_div(uint32_t n, const FastDiv& f) { return uint32_t((uint64_t(n) * f.m) >> f.k); }

// A 64-token tile is one frame of a block, tile row k = 8 * y + x. A 32x32 score accumulator of
// the 32-row tile kt of such a tile (the MFMA result layout) holds, in item v of a lane with lane
// half hi, tile row kt*32 + 8*(v/4) + 4*hi + v%4. Items whose token lies outside the grid of a
// partial block (rows x cols inside) are set to -inf, so they take no probability mass.
template <class V>
LCSA_HD void mask_partial_tile(V& s, int kt, int hi, int rows, int cols) {
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int y = kt * 4 + v / 4, x = 4 * hi + v % 4;
    if (!(y < rows && x < cols)) s[v] = -INFINITY;
  }
}

// Token-window mask of the same accumulator layout for a key tile whose first token sits at row h0,
// column w0 of the grid, for a lane whose query token sees rows [lo_h, hi_h] and columns [lo_w, hi_w]
// (also masks tokens past the grid edge, which lie outside every window).
template <class V>
LCSA_HD void mask_window_tile(V& s, int kt, int hi, int h0, int w0, int lo_h, int hi_h, int lo_w, int hi_w) {
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int hk = h0 + kt * 4 + v / 4, wk = w0 + 4 * hi + v % 4;
    if (!(hk >= lo_h && hk <= hi_h && wk >= lo_w && wk <= hi_w)) s[v] = -INFINITY;
  }
}

// The same token-window test with the roles swapped (the dK/dV layout: accumulator rows are query
// tokens, the lane holds one key token at (hk, wk)): item v's query token sits at row qh0 + kt*4 + v/4,
// column qw0 + 4*hi + v%4; it is masked when it lies outside the grid or its window misses the key.
template <class V>
LCSA_HD void mask_window_tile_q(V& s, int kt, int hi, int qh0, int qw0, int hk, int wk, const Geom& g) {
  const bool pres = g.win_mode == kWinTokenPreserving;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int hq = qh0 + kt * 4 + v / 4, wq = qw0 + 4 * hi + v % 4;
    int lh, hh, lw, hw2;
    tok_range(pres, hq, g.H, g.wth, &lh, &hh);
    tok_range(pres, wq, g.W, g.wtw, &lw, &hw2);
    if (!(hq < g.H && wq < g.W && hk >= lh && hk <= hh && wk >= lw && wk <= hw2)) s[v] = -INFINITY;
  }
}

// Whether key block (hb, wb) lies wholly inside the window of every token of query block (qhb, qwb):
// the bounds are monotone, so the last query row / column bounds the start and the first the end.
LCSA_HD bool block_seen_whole(const Geom& g, int qhb, int qwb, int hb, int wb) {
  const bool pres = g.win_mode == kWinTokenPreserving;
  int lo_last, hi_last, lo_first, hi_first;
  tok_range(pres, kBlkH * qhb + block_rows(g, qhb) - 1, g.H, g.wth, &lo_last, &hi_last);
  tok_range(pres, kBlkH * qhb, g.H, g.wth, &lo_first, &hi_first);
  if (!(kBlkH * hb >= lo_last && kBlkH * hb + kBlkH - 1 <= hi_first)) return false;
  tok_range(pres, kBlkW * qwb + block_cols(g, qwb) - 1, g.W, g.wtw, &lo_last, &hi_last);
  tok_range(pres, kBlkW * qwb, g.W, g.wtw, &lo_first, &hi_first);
  return kBlkW * wb >= lo_last && kBlkW * wb + kBlkW - 1 <= hi_first;
}

// Order of workgroups that each take `rows_per_wg` consecutive rows of the (batch, head)-major query
// blocks (`nqb` per head). Hardware deals workgroup n to XCD n % 8 (local index n / 8). Each XCD
// takes a contiguous range of the work, as equal in length as the count allows, so the workgroups that
// share a head's K and V share one L2. Within its range an XCD starts at the first head boundary when
// the part from there on is at least as long as the head tail before it, and wraps round to that tail:
// the workgroups that start together then come from one head. With `descending`, each head's piece is
// walked from its last row back: under the causal mask later rows keep more key blocks, so the long
// workgroups start first and the short ones fill the end.
LCSA_HD int xcd_work_order(int n, int nwg, int rows_per_wg, int nqb, bool descending) {
  const int x = n % 8, l = n / 8;
  const int q = nwg / 8, rem = nwg % 8;
  const int c = q + (x < rem ? 1 : 0);
  const int s = x * q + (x < rem ? x : rem);
  const int rb = ((rows_per_wg * s + nqb - 1) / nqb) * nqb;  // first head-start row at or after s
  int b = (rb + rows_per_wg - 1) / rows_per_wg;               // the workgroup holding it
  if (b > s + c) b = s + c;
  const int off = (s + c - b >= b - s) ? b - s : 0;
  const int k = off + l;
  const int g0 = s + (k >= c ? k - c : k);
  if (!descending) return g0;
  // mirror g0 inside its piece of one head: [b, s + c) or [s, b), cut at head boundaries
  const int h = (rows_per_wg * g0) / nqb;
  const int hs = (h * nqb + rows_per_wg - 1) / rows_per_wg, he = ((h + 1) * nqb + rows_per_wg - 1) / rows_per_wg;
  const int lo = g0 >= b ? (hs > b ? hs : b) : (hs > s ? hs : s);
  const int hi = g0 >= b ? (he < s + c ? he : s + c) : (he < b ? he : b);
  return lo + hi - 1 - g0;
}

LCSA_HD int n_visible(const Geom& g, int i) {
  int h0, h1, w0, w1;
  const int tb = qblock_window(g, i, &h0, &h1, &w0, &w1);
  return (tb + 1) * (h1 - h0 + 1) * (w1 - w0 + 1);
}

}  // namespace lcsa
