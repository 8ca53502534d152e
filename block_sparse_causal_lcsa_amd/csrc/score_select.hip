// lcsa_score_select: coarse block map + causal/window mask + per-row Top-K -> CSR column lists
// (FlashVSR summary, sec. 2.2: a coarse block-to-block attention map from the pooled features,
// the Top-K most relevant block pairs are kept; sec. 2.3: the local spatial window).
//
// One workgroup per (batch, head, tile of kRows consecutive query blocks), one wave per query block.
//  1. Candidates. The tile's candidate set is the union of its rows' visible sets: the temporal
//     blocks up to the last one any row sees, times the smallest rectangle of block rows and columns
//     holding every row's window. It is enumerated in ascending key-block index (temporal block, then
//     block row, then block column), so no row holds more than its tile's union, whatever the number
//     of key blocks; a row's own mask is applied to the union when the scores are stored.
//  2. Scores: s_ij = scale * <qbar_i, kbar_j> in fp64 (the fp32 pooled features widen exactly), with
//     v_mfma_f64_4x4x4 in its 4-block form: one instruction scores the tile's 4 rows against 16
//     candidates over 4 channels. Scores sit in LDS, [row][candidate], -inf where not visible.
//  3. Selection, one wave per row: scores map to order-preserving 64-bit keys held in registers; a
//     bisection over the key range, counting the keys at or above the midpoint with one ballot and
//     popcount per register, finds the key T of the K_i-th largest score (it stops early when some
//     threshold leaves exactly K_i keys at or above it). Keys above T are kept, keys equal to T lowest
//     index first; kept indices are emitted ascending with ballot prefix sums.
// The selection is exact for the fp64 scores: the largest K_i scores, exact ties to the lower j.
// Workgroups are ordered so that each XCD (hardware deals workgroup n to XCD n mod 8) takes one
// contiguous run of the (batch, head)-major tiles: a head's tiles share one or two XCDs' L2, which
// then serves its pooled K to all of them, and every XCD gets the same number of tiles.
#include <hip/hip_runtime.h>

#include <math.h>

#include <atomic>

#include "lcsa_internal.h"

namespace lcsa {
namespace {

constexpr int kXcds = 8;
constexpr int kLdsBytes = 160 * 1024;  // LDS per workgroup on gfx950

struct SelArgs {
  const float* qp;     // [B*Hh, nqb, D]
  const float* kp;     // [B*Hh, nkb, D]
  const int32_t* row_ptr;
  int32_t* col_idx;    // [B*Hh, nnz]
  double* dbg;         // [B*Hh, nqb, nkb] or null
  Geom g;
  int32_t nnz;
  int32_t bh;          // batch * heads
  int32_t tiles;       // query-block tiles per (batch, head)
  int32_t nwg;         // bh * tiles workgroups
  int32_t ld;          // LDS row stride of the scores, in doubles
  double scale;
  FastDiv div_bpt, div_wb;  // division by g.bpt and g.Wb
};

// A tile's candidate set: temporal blocks [0, nt), block rows [h0, h0 + nh), columns [w0, w0 + nw).
struct Union {
  int nt, h0, nh, w0, nw;
  LCSA_HD int size() const { return nt * nh * nw; }
};

LCSA_HD Union tile_union(const Geom& g, int r0, int rows) {
  Union u{0, 1 << 30, 0, 1 << 30, 0};
  int h1 = -1, w1 = -1;
  for (int r = 0; r < rows; ++r) {
    int a0, a1, b0, b1;
    const int tb = qblock_window(g, r0 + r, &a0, &a1, &b0, &b1);
    u.nt = tb + 1 > u.nt ? tb + 1 : u.nt;
    u.h0 = a0 < u.h0 ? a0 : u.h0;
    u.w0 = b0 < u.w0 ? b0 : u.w0;
    h1 = a1 > h1 ? a1 : h1;
    w1 = b1 > w1 ? b1 : w1;
  }
  u.nh = h1 - u.h0 + 1;
  u.nw = w1 - u.w0 + 1;
  return u;
}

__device__ __forceinline__ uint64_t order_key(double s) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(s == 0.0 ? 0.0 : s));
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// Maximum of x over the wave: row shifts give each lane the maximum of its row so far, the broadcasts of
// lanes 15 and 31 carry it across rows, and lane 63 ends with the whole wave's maximum. Lanes whose
// source lies outside the row take 0, the identity.
__device__ __forceinline__ uint32_t wave_max(uint32_t x) {
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x111, 0xf, 0xf, false)));  // row_shr:1
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x112, 0xf, 0xf, false)));  // row_shr:2
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x114, 0xf, 0xf, false)));  // row_shr:4
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x118, 0xf, 0xf, false)));  // row_shr:8
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x142, 0xa, 0xf, false)));  // row_bcast:15
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0, int(x), 0x143, 0xc, 0xf, false)));  // row_bcast:31
  return __builtin_amdgcn_readlane(x, 63);
}

// floor(u / d) for 0 <= u < 2^22 and 1 <= d, with rcp = 1.0f / d: the float product is within 1/2 of
// the quotient, so one correction either way makes it exact.
__device__ __forceinline__ int udiv_small(int u, int d, float rcp) {
  int q = int(float(u) * rcp);
  q -= q * d > u;
  q += (q + 1) * d <= u;
  return q;
}

// Position of candidate u in a tile's union: temporal block t, block row hb, block column wb.
struct UnionDiv {
  int hw;
  float rcp_hw, rcp_nw;
};

__device__ __forceinline__ void union_pos(const Union& un, const UnionDiv& ud, int u, int* t, int* hb, int* wb) {
  *t = udiv_small(u, ud.hw, ud.rcp_hw);
  const int rem = u - *t * ud.hw;
  const int dh = udiv_small(rem, un.nw, ud.rcp_nw);
  *hb = un.h0 + dh;
  *wb = un.w0 + rem - dh * un.nw;
}

// Key block of candidate u of a tile's union.
__device__ __forceinline__ int union_block(const Geom& g, const Union& un, const UnionDiv& ud, int u) {
  int t, hb, wb;
  union_pos(un, ud, u, &t, &hb, &wb);
  return (t * g.Hb + hb) * g.Wb + wb;
}

// Keys of a row's candidates u = lane + 64 m (m < SLOTS) as high and low 32-bit halves; 0 for masked
// entries and u >= U, below every candidate key (a candidate's high half is at least 2^20). SLOTS = 0:
// the row is longer than the registers hold and every pass reads the scores from LDS again.
template <int SLOTS>
struct RowKeys {
  uint32_t hi[SLOTS > 0 ? SLOTS : 1], lo[SLOTS > 0 ? SLOTS : 1];
};

// Count of this wave's candidates whose key has high half >= th (PHASE 0), or high half == th and low
// half >= tl (PHASE 1). th >= 1, so masked entries never count.
template <int SLOTS, int PHASE>
__device__ __forceinline__ int count_keys(const RowKeys<SLOTS>& rk, const double* srow, int U, int lane, uint32_t th,
                                          uint32_t tl) {
  int c = 0;
  if constexpr (SLOTS > 0) {
#pragma unroll
    for (int m = 0; m < SLOTS; ++m)
      c += __popcll(__ballot(PHASE == 0 ? rk.hi[m] >= th : (rk.hi[m] == th && rk.lo[m] >= tl)));
  } else {
    for (int u0 = 0; u0 < U; u0 += 64) {
      const double x = u0 + lane < U ? srow[u0 + lane] : -INFINITY;
      const uint64_t k = x != -INFINITY ? order_key(x) : 0;
      const uint32_t h = uint32_t(k >> 32), l = uint32_t(k);
      c += __popcll(__ballot(PHASE == 0 ? h >= th : (h == th && l >= tl)));
    }
  }
  return c;
}

// Largest t in [lo, hi] with count(t) >= need, given count(lo) >= need (count non-increasing in t);
// stops early at a t whose count is exactly `need` (then *exact is set). Uniform scalar loop.
template <typename F>
__device__ __forceinline__ uint32_t bisect(uint32_t lo, uint32_t hi, int need, bool* exact, F&& count) {
  *exact = false;
  while (lo < hi) {
    const uint32_t mid = lo + (hi - lo) / 2 + 1;
    const int c = count(mid);
    if (c == need) {
      *exact = true;
      return mid;
    }
    if (c > need) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

template <int D, int kRows, int SLOTS, bool WIDE>
__global__ __launch_bounds__(64 * kRows) void score_select_kernel(SelArgs a) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  extern __shared__ double S[];  // [kRows][a.ld] scores
  const Geom& g = a.g;
  // XCD-contiguous order over the (batch, head)-major tiles
  int wg = blockIdx.x;
  const int n8 = (a.nwg / kXcds) * kXcds;
  if (wg < n8) wg = (wg % kXcds) * (a.nwg / kXcds) + wg / kXcds;
  const int bh = wg / a.tiles;
  const int r0 = (wg - bh * a.tiles) * kRows;
  const int rows = min(kRows, g.nqb - r0);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // this wave's row of the selection: its CSR range, loaded early (uniform scalar loads)
  const int i_sel = r0 + (wave < rows ? wave : 0);
  const int rp_beg = __builtin_amdgcn_readfirstlane(a.row_ptr[i_sel]);
  const int K = __builtin_amdgcn_readfirstlane(a.row_ptr[i_sel + 1]) - rp_beg;

  // ---- scores. v_mfma_f64_4x4x4f64, 4 blocks: block b (0..3) multiplies A_b (4 rows x 4 k) by
  // B_b (4 k x 4 columns). A_b[i][k] comes from lane 16k + 4b + i, B_b[k][j] from lane 16k + 4b + j,
  // and D_b[i][j] lands in lane 16i + 4b + j. Every block takes the tile's 4 rows as A, block b takes
  // candidates 4b..4b+3 of the column tile as B: one instruction = 4 rows x 16 candidates x 4 channels.
  // Channel order within the dot product: step s (0..D/4-1) and k give channel (D/4) k + s, so each lane
  // reads one contiguous run of D/4 channels of its row and of its candidate.
  constexpr int KR = D / 4;  // channels per lane
  const int lk = lane >> 4;
  const int qi = lane & 3;   // A row of this lane
  const int lc = lane & 15;  // B column (candidate within the column tile) of this lane
  float4 qf[KR / 4];
  {
    const int qrow = r0 + (qi < rows ? qi : 0);
    const float4* src = reinterpret_cast<const float4*>(a.qp + (int64_t(bh) * g.nqb + qrow) * D + KR * lk);
#pragma unroll
    for (int v = 0; v < KR / 4; ++v) qf[v] = src[v];
  }
  // each row's own window (candidate test when the scores are stored) and the tile's union: lane r
  // works out row r0 + r (lanes past the tile repeat its first row), the rows are then read back
  int tbi[kRows], h0[kRows], h1[kRows], w0[kRows], w1[kRows];
  Union un{0, 1 << 30, 0, 1 << 30, 0};
  {
    const uint32_t ir = uint32_t(r0 + (lane < rows ? lane : 0));
    const uint32_t tr = fast_div(ir, a.div_bpt), rem = ir - tr * uint32_t(g.bpt);
    const uint32_t hb = fast_div(rem, a.div_wb), wb = rem - hb * uint32_t(g.Wb);
    int lh0, lh1, lw0, lw1;
    qblock_window_at(g, int(hb), int(wb), &lh0, &lh1, &lw0, &lw1);
    const int ltb = g.q_tb0 + int(tr);
    int uh1 = -1, uw1 = -1;
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      tbi[r] = __builtin_amdgcn_readlane(ltb, r);
      h0[r] = __builtin_amdgcn_readlane(lh0, r);
      h1[r] = __builtin_amdgcn_readlane(lh1, r);
      w0[r] = __builtin_amdgcn_readlane(lw0, r);
      w1[r] = __builtin_amdgcn_readlane(lw1, r);
      un.nt = max(un.nt, tbi[r] + 1);
      un.h0 = min(un.h0, h0[r]);
      un.w0 = min(un.w0, w0[r]);
      uh1 = max(uh1, h1[r]);
      uw1 = max(uw1, w1[r]);
    }
    un.nh = uh1 - un.h0 + 1;
    un.nw = uw1 - un.w0 + 1;
  }
  const UnionDiv ud{un.nh * un.nw, 1.0f / float(un.nh * un.nw), 1.0f / float(un.nw)};
  const int U = un.size();
  const int nct = (U + 15) / 16;  // 16-candidate column tiles
  const float* kmat = a.kp + int64_t(bh) * g.nkb * D;
  auto load_col = [&](int ct, float4 (&kb)[KR / 4]) __attribute__((always_inline)) {
    const int u = min(16 * ct + lc, U - 1);
    const float4* src = reinterpret_cast<const float4*>(kmat + int64_t(union_block(g, un, ud, u)) * D + KR * lk);
#pragma unroll
    for (int v = 0; v < KR / 4; ++v) kb[v] = src[v];
  };
  // this wave's column tiles ct = wave + kRows n; the loads of PF of them are in flight at a time
  constexpr int PF = 4;
  float4 kb[PF][KR / 4];
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (wave + kRows * p < nct) load_col(wave + kRows * p, kb[p]);
  double qa[KR];
#pragma unroll
  for (int v = 0; v < KR / 4; ++v) {
    qa[4 * v] = qf[v].x; qa[4 * v + 1] = qf[v].y; qa[4 * v + 2] = qf[v].z; qa[4 * v + 3] = qf[v].w;
  }
  const int orow = lane >> 4;  // result row of this lane
  for (int n = 0; wave + kRows * n < nct; n += PF) {
#pragma unroll
    for (int p = 0; p < PF; ++p) {
      const int ct = wave + kRows * (n + p);
      if (ct >= nct) break;
      double acc[4] = {0.0, 0.0, 0.0, 0.0};  // four independent chains, summed in a fixed order
      if constexpr (WIDE) {
        // the whole column tile is widened first, into registers of its own: widening each value just
        // before its MFMA reuses one register pair, and an MFMA still reading it holds up the next
        // widening, so the chains run one MFMA at a time (about 3x slower). It costs 64 registers,
        // hence one wave per SIMD; launched only when every workgroup has a CU of its own.
        double kd[KR];
#pragma unroll
        for (int v = 0; v < KR / 4; ++v) {
          kd[4 * v] = kb[p][v].x;
          kd[4 * v + 1] = kb[p][v].y;
          kd[4 * v + 2] = kb[p][v].z;
          kd[4 * v + 3] = kb[p][v].w;
        }
#pragma unroll
        for (int v = 0; v < KR / 4; ++v)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[e] = __builtin_amdgcn_mfma_f64_4x4x4f64(qa[4 * v + e], kd[4 * v + e], acc[e], 0, 0, 0);
      } else {
        // half a tile at a time (32 registers), so two workgroups still fit a CU
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          double kd[KR / 2];
#pragma unroll
          for (int v = 0; v < KR / 8; ++v) {
            const float4 f = kb[p][half * (KR / 8) + v];
            kd[4 * v] = f.x;
            kd[4 * v + 1] = f.y;
            kd[4 * v + 2] = f.z;
            kd[4 * v + 3] = f.w;
          }
#pragma unroll
          for (int v = 0; v < KR / 8; ++v)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[e] = __builtin_amdgcn_mfma_f64_4x4x4f64(qa[4 * (half * (KR / 8) + v) + e], kd[4 * v + e], acc[e],
                                                          0, 0, 0);
        }
      }
      if (ct + kRows * PF < nct) load_col(ct + kRows * PF, kb[p]);
      const double sc = ((acc[0] + acc[1]) + (acc[2] + acc[3])) * a.scale;
      const int u = 16 * ct + lc;
      if (u < U && orow < kRows) {
        int t, hb, wb;
        union_pos(un, ud, u, &t, &hb, &wb);
        bool vis = false;
#pragma unroll
        for (int r = 0; r < kRows; ++r)
          if (r == orow) vis = r < rows && t <= tbi[r] && hb >= h0[r] && hb <= h1[r] && wb >= w0[r] && wb <= w1[r];
        S[orow * a.ld + u] = vis ? sc : -INFINITY;
      }
    }
  }
  __syncthreads();

  // ---- selection: wave rl selects row r0 + rl
  const int rl = wave;
  if (rl >= rows) return;
  const int i = r0 + rl;
  const double* srow = S + rl * a.ld;
  if (a.dbg) {
    double* drow = a.dbg + (int64_t(bh) * g.nqb + i) * g.nkb;
    const int hw = un.nh * un.nw;
    for (int j = lane; j < g.nkb; j += 64) {
      const int t = j / g.bpt, rem = j - t * g.bpt;
      const int hb = rem / g.Wb, wb = rem - (rem / g.Wb) * g.Wb;
      const bool in = t < un.nt && hb >= un.h0 && hb < un.h0 + un.nh && wb >= un.w0 && wb < un.w0 + un.nw;
      drow[j] = in ? srow[t * hw + (hb - un.h0) * un.nw + (wb - un.w0)] : -INFINITY;
    }
  }
  int32_t* out = a.col_idx + int64_t(bh) * a.nnz + rp_beg;
  RowKeys<SLOTS> rk;
  int ncand = 0;
  if constexpr (SLOTS > 0) {
#pragma unroll
    for (int m = 0; m < SLOTS; ++m) {
      const int u = lane + 64 * m;
      const double x = u < U ? srow[u] : -INFINITY;
      const uint64_t k = x != -INFINITY ? order_key(x) : 0;
      rk.hi[m] = uint32_t(k >> 32);
      rk.lo[m] = uint32_t(k);
      ncand += __popcll(__ballot(k != 0));
    }
  } else {
    ncand = count_keys<SLOTS, 0>(rk, srow, U, lane, 1, 0);
  }
  // The kept set: keys above the threshold (th, tl), plus the first `ties` keys equal to it (by
  // index); ties == 0 means every key >= (th, tl) and no other. First the high halves are bisected;
  // only when the K_i-th key shares its high half with a key that is not kept (scores within about
  // 2^-20 relative of each other) are the low halves bisected among that high half.
  const int need = min(K, ncand);
  uint32_t th = 1, tl = 0;
  int ties = 0;
  if (need < ncand) {
    // the high halves span [hmin, hmax]; the bisection starts from that range
    uint32_t hmin = 1, hmax = ~0u;
    if constexpr (SLOTS > 0) {
      uint32_t mx = 0, mn = 0;  // mn holds ~(smallest candidate high half)
#pragma unroll
      for (int m = 0; m < SLOTS; ++m) {
        mx = max(mx, rk.hi[m]);
        mn = max(mn, rk.hi[m] ? ~rk.hi[m] : 0u);
      }
      hmax = wave_max(mx);
      hmin = ~wave_max(mn);
    }
    bool exact;
    th = bisect(hmin, hmax, need, &exact,
                [&](uint32_t t) { return count_keys<SLOTS, 0>(rk, srow, U, lane, t, 0); });
    if (!exact) {
      const int above = th == ~0u ? 0 : count_keys<SLOTS, 0>(rk, srow, U, lane, th + 1, 0);
      const int need2 = need - above;  // >= 1 of the keys with high half th
      tl = bisect(0u, ~0u, need2, &exact,
                  [&](uint32_t t) { return count_keys<SLOTS, 1>(rk, srow, U, lane, th, t); });
      if (!exact) {
        const int above2 = tl == ~0u ? 0 : count_keys<SLOTS, 1>(rk, srow, U, lane, th, tl + 1);
        ties = need2 - above2;
      }
    }
  }
  // emit ascending
  const uint64_t T = (uint64_t(th) << 32) | tl;
  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  int written = 0, seen = 0;
  auto emit = [&](int u, uint64_t k) __attribute__((always_inline)) {
    const bool c = k != 0;
    const bool tie = c & (ties > 0) & (k == T);
    const uint64_t tb = __ballot(tie);
    const bool sel = c & (ties > 0 ? (k > T || (tie && seen + __popcll(tb & lt_mask) < ties)) : (k >= T));
    seen += __popcll(tb);
    const uint64_t sb = __ballot(sel);
    if (sel) out[written + __popcll(sb & lt_mask)] = union_block(g, un, ud, u);
    written += __popcll(sb);
  };
  if constexpr (SLOTS > 0) {
#pragma unroll
    for (int m = 0; m < SLOTS; ++m) {
      if (64 * m >= U) break;
      emit(lane + 64 * m, (uint64_t(rk.hi[m]) << 32) | rk.lo[m]);
    }
  } else {
    for (int u0 = 0; u0 < U; u0 += 64) {
      const double x = u0 + lane < U ? srow[u0 + lane] : -INFINITY;
      emit(u0 + lane, x != -INFINITY ? order_key(x) : 0);
    }
  }
  for (int s = written + lane; s < K; s += 64) out[s] = -1;  // only if row_ptr asks for > n_i
}

// The dynamic-LDS limit of each kernel instantiation is raised once per device (to the whole LDS),
// not on every call, so that launches can be captured into a HIP graph.
constexpr int kMaxDevices = 64;

// Compute units of the current device (cached per device).
int device_cus(int dev) {
  static std::atomic<int> cus[kMaxDevices];
  int n = cus[dev].load(std::memory_order_acquire);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 1 << 30;
    cus[dev].store(n, std::memory_order_release);
  }
  return n;
}

template <int D, int kRows, int SLOTS, bool WIDE>
lcsa_status launch_one(SelArgs a, size_t lds, int dev, hipStream_t s) {
  static std::atomic<uint64_t> raised[kMaxDevices];
  if (raised[dev].load(std::memory_order_acquire) == 0) {
    const lcsa_status st =
        hip_status(hipFuncSetAttribute(reinterpret_cast<const void*>(&score_select_kernel<D, kRows, SLOTS, WIDE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes),
                   "lcsa_score_select LDS size");
    if (st != LCSA_OK) return st;
    raised[dev].store(1, std::memory_order_release);
  }
  score_select_kernel<D, kRows, SLOTS, WIDE><<<a.nwg, 64 * kRows, lds, s>>>(a);
  return LCSA_OK;
}

template <int D, int kRows, int SLOTS>
lcsa_status launch(SelArgs a, int max_union, hipStream_t s) {
  int dev = 0;
  lcsa_status st = hip_status(hipGetDevice(&dev), "lcsa_score_select device");
  if (st != LCSA_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(LCSA_ERR_UNSUPPORTED, "lcsa_score_select: device %d", dev);
  a.ld = ((max_union + 15) / 16) * 16 + 2;  // the pad spreads the 4 rows of a store over the banks
  const size_t lds = size_t(kRows) * a.ld * sizeof(double);
  a.tiles = (a.g.nqb + kRows - 1) / kRows;
  a.nwg = a.bh * a.tiles;
  // the widened-tile form when the grid is one workgroup per CU or less (small problems, where the
  // scoring chain is the critical path); otherwise two workgroups per CU matter more
  if constexpr (kRows == 4 && SLOTS > 0 && SLOTS <= 8) {
    if (a.nwg <= device_cus(dev)) return launch_one<D, kRows, SLOTS, true>(a, lds, dev, s);
  }
  return launch_one<D, kRows, SLOTS, false>(a, lds, dev, s);
}

// Register slots of 64 candidates for the longest row: 4, 8, 16 or 32; beyond 2048 candidates the
// selection reads the scores from LDS on every pass (0).
template <int D, int kRows>
lcsa_status launch_slots(const SelArgs& a, int max_union, hipStream_t s) {
  const int slots = (max_union + 63) / 64;
  if (slots <= 4) return launch<D, kRows, 4>(a, max_union, s);
  if (slots <= 8) return launch<D, kRows, 8>(a, max_union, s);
  if (slots <= 16) return launch<D, kRows, 16>(a, max_union, s);
  if (slots <= 32) return launch<D, kRows, 32>(a, max_union, s);
  return launch<D, kRows, 0>(a, max_union, s);
}

// LDS bytes a workgroup of `rows` rows needs for a union of `u` candidates.
size_t lds_need(int rows, int u) { return size_t(rows) * (((u + 15) / 16) * 16 + 2) * sizeof(double); }

}  // namespace
}  // namespace lcsa

using namespace lcsa;

extern "C" lcsa_status lcsa_score_select(const lcsa_problem* p, const float* q_pooled, const float* k_pooled,
                                         const int32_t* row_ptr, int32_t* col_idx, double* scores_dbg,
                                         void* stream) {
  Geom g;
  lcsa_status st = validate_problem(p, &g);
  if (st != LCSA_OK) return st;
  if (!q_pooled || !k_pooled || !row_ptr || !col_idx)
    return fail(LCSA_ERR_INVALID, "lcsa_score_select: NULL input or output pointer");
  if (reinterpret_cast<uintptr_t>(q_pooled) % 16 || reinterpret_cast<uintptr_t>(k_pooled) % 16 ||
      reinterpret_cast<uintptr_t>(row_ptr) % 4 || reinterpret_cast<uintptr_t>(col_idx) % 4 ||
      reinterpret_cast<uintptr_t>(scores_dbg) % 8)
    return fail(LCSA_ERR_INVALID, "lcsa_score_select: misaligned pointer");
  int32_t nnz = 0;
  if ((st = lcsa_csr_layout(p, nullptr, nullptr, &nnz, nullptr)) != LCSA_OK) return st;
  // the largest candidate union over the tiles of 4 rows, and over single rows (the fallback for
  // unions beyond the LDS)
  int max4 = 0, max1 = 0;
  for (int r0 = 0; r0 < g.nqb; r0 += 4) {
    const int u = tile_union(g, r0, g.nqb - r0 < 4 ? g.nqb - r0 : 4).size();
    max4 = u > max4 ? u : max4;
  }
  for (int i = 0; i < g.nqb; ++i) {
    const int u = tile_union(g, i, 1).size();
    max1 = u > max1 ? u : max1;
  }
  SelArgs a{};
  a.qp = q_pooled;
  a.kp = k_pooled;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.dbg = scores_dbg;
  a.g = g;
  a.nnz = nnz;
  a.bh = p->batch * p->heads;
  a.scale = static_cast<double>(p->scale);
  a.div_bpt = make_fastdiv(static_cast<uint32_t>(g.bpt));
  a.div_wb = make_fastdiv(static_cast<uint32_t>(g.Wb));
  // validate_problem bounds B * Hh * nkb by 2^30, so B * Hh * nqb workgroups fit an int
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const bool four = lds_need(4, max4) <= size_t(kLdsBytes);
  if (!four && lds_need(1, max1) > size_t(kLdsBytes))
    return fail(LCSA_ERR_UNSUPPORTED, "lcsa_score_select: %d candidate key blocks for one query block exceed the %d "
                "that LDS holds", max1, kLdsBytes / 8 - 18);
  if (p->head_dim == 128) st = four ? launch_slots<128, 4>(a, max4, s) : launch_slots<128, 1>(a, max1, s);
  else st = four ? launch_slots<64, 4>(a, max4, s) : launch_slots<64, 1>(a, max1, s);
  if (st != LCSA_OK) return st;
  return hip_status(hipGetLastError(), "lcsa_score_select launch");
}
