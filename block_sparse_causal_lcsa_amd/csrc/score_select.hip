// lcsa_score_select: coarse block map + causal/window mask + per-row Top-K -> CSR column lists
// (FlashVSR summary, sec. 2.2: a coarse block-to-block attention map from the pooled features,
// the Top-K most relevant block pairs are kept; sec. 2.3: the local spatial window).
//
// One workgroup (16 or 4 waves) per (batch, head, tile of 16 or 4 query blocks).
//  1. Scores: s_ij = scale * <qbar_i, kbar_j> for the tile's 16 rows against every key block up to
//     the last temporal block the tile can see, as fp64 MFMA 16x16x4 tiles (the pooled fp32
//     features are widened exactly). Column tiles with no visible entry are skipped. Rows of 16
//     fp64 scores live in LDS, -inf where the key block is not visible.
//  2. Selection, one wave per row (all 16 rows in parallel): scores map to order-preserving 64-bit keys; a most-significant-
//     bit-first radix select over the wave's candidates (ballot + popcount per bit) finds the key of
//     the K_i-th largest score and how many of the keys equal to it are still needed; equal keys are
//     taken lowest index first. Kept indices are emitted in ascending order with ballot prefix sums.
// The selection is exact for the fp64 scores: the largest K_i scores, exact ties to the lower j.
#include <hip/hip_runtime.h>

#include <math.h>

#include <atomic>

#include "lcsa_internal.h"

namespace lcsa {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

// ROWS query blocks per workgroup, one wave each: 16 shares each loaded pooled-K tile among 16
// rows; 4 gives four times the workgroups when a problem has too few rows to fill the chip.
constexpr int kRowsWide = 16, kRowsNarrow = 4;
constexpr int kMaxCols = 1248;            // key blocks one row can hold in LDS
constexpr int kMaxSlots = (kMaxCols + 63) / 64;
constexpr int kLdsPad = 2;

struct SelArgs {
  const float* qp;     // [B*Hh, nqb, D]
  const float* kp;     // [B*Hh, nkb, D]
  const int32_t* row_ptr;
  int32_t* col_idx;    // [B*Hh, nnz]
  double* dbg;         // [B*Hh, nqb, nkb] or null
  Geom g;
  int32_t nnz;
  int32_t ld;          // LDS row stride in doubles
  double scale;
};

__device__ __forceinline__ bool is_visible(const Geom& g, int tbi, int h0, int h1, int w0, int w1, int j) {
  const int tbj = j / g.bpt, rem = j - (j / g.bpt) * g.bpt;
  const int hb = rem / g.Wb, wb = rem - (rem / g.Wb) * g.Wb;
  return tbj <= tbi && hb >= h0 && hb <= h1 && wb >= w0 && wb <= w1;
}

// Inclusive prefix sum over the 64 lanes of a wave (lane order), with DPP row shifts inside each
// 16-lane row and row broadcasts across rows.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false); // row_bcast:15 into rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false); // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ uint64_t order_key(double s) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(s == 0.0 ? 0.0 : s));
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

template <int D, int SLOTS, int kRows>
__global__ __launch_bounds__(64 * kRows) void score_select_kernel(SelArgs a) {
  extern __shared__ double S[];  // [kRows][a.ld]
  const Geom& g = a.g;
  const int tiles = (g.nqb + kRows - 1) / kRows;
  const int bh = blockIdx.x / tiles;
  const int r0 = (blockIdx.x - bh * tiles) * kRows;
  const int rows = min(kRows, g.nqb - r0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;

  // key blocks up to the last temporal block visible from the tile's last row
  const int tb_last = g.q_tb0 + (r0 + rows - 1) / g.bpt;
  const int ncol = min((tb_last + 1) * g.bpt, g.nkb);
  const int nct = (ncol + 15) / 16;

  const float* qrow = a.qp + (int64_t(bh) * g.nqb + r0 + min(lr, rows - 1)) * D;
  const float* kmat = a.kp + int64_t(bh) * g.nkb * D;

  // A operand (16 query rows x 4 channels per step). Lane (lr, lg) supplies row lr; k-step
  // 4m+e covers channels 16m + 4*lg + e, so each lane reads float4s; B uses the same mapping.
  float4 qa[D / 16];
#pragma unroll
  for (int m = 0; m < D / 16; ++m) qa[m] = *reinterpret_cast<const float4*>(qrow + 16 * m + 4 * lg);

  // window of the 4 output rows this lane holds in the MFMA result (rows lg + 4*rr)
  int tbi[4], h0[4], h1[4], w0[4], w1[4];
  bool rv[4];
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int i = r0 + lg + 4 * rr;
    rv[rr] = i < g.nqb && (lg + 4 * rr) < rows;
    tbi[rr] = qblock_window(g, rv[rr] ? i : r0, &h0[rr], &h1[rr], &w0[rr], &w1[rr]);
  }

  for (int ct = wave; ct < nct; ct += kRows) {
    const int j = ct * 16 + lr;
    bool vis[4];
    bool any = false;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      vis[rr] = rv[rr] && j < ncol && is_visible(g, tbi[rr], h0[rr], h1[rr], w0[rr], w1[rr], j);
      any |= vis[rr];
    }
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
    if (__any(any)) {
      const float* krow = kmat + int64_t(min(j, ncol - 1)) * D;
      // four independent accumulation chains (channel e of each float4), summed in a fixed order
      f64x4 c[4] = {acc, acc, acc, acc};
#pragma unroll
      for (int m = 0; m < D / 16; ++m) {
        const float4 kb = *reinterpret_cast<const float4*>(krow + 16 * m + 4 * lg);
        c[0] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)qa[m].x, (double)kb.x, c[0], 0, 0, 0);
        c[1] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)qa[m].y, (double)kb.y, c[1], 0, 0, 0);
        c[2] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)qa[m].z, (double)kb.z, c[2], 0, 0, 0);
        c[3] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)qa[m].w, (double)kb.w, c[3], 0, 0, 0);
      }
      acc = (c[0] + c[1]) + (c[2] + c[3]);
    }
    // result item rr of lane (lr, lg) is D[row lg + 4*rr][col lr]
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      if (lg + 4 * rr < kRows) S[(lg + 4 * rr) * a.ld + j] = vis[rr] ? acc[rr] * a.scale : -INFINITY;
  }
  __syncthreads();

  const uint64_t lt_mask = (uint64_t(1) << lane) - 1;
  for (int rl = wave; rl < rows; rl += kRows) {
    const int i = r0 + rl;
    const double* srow = S + rl * a.ld;
    if (a.dbg) {
      double* drow = a.dbg + (int64_t(bh) * g.nqb + i) * g.nkb;
      for (int j = lane; j < g.nkb; j += 64) drow[j] = j < ncol ? srow[j] : -INFINITY;
    }
    const int K = a.row_ptr[i + 1] - a.row_ptr[i];
    int32_t* out = a.col_idx + int64_t(bh) * a.nnz + a.row_ptr[i];

    // non-candidates (masked, beyond the row) get key 0, below every candidate's key; the loops
    // below are branch-free over a fixed slot count
    uint64_t key[SLOTS];
    int ncand = 0;
#pragma unroll
    for (int m = 0; m < SLOTS; ++m) {
      const int j = lane + 64 * m;
      const double s = j < ncol ? srow[j] : -INFINITY;
      const bool c = s != -INFINITY;
      key[m] = c ? order_key(s) : 0;
      ncand += __popcll(__ballot(c));
    }
    int need = min(K, ncand);
    uint64_t prefix = 0, mask = 0;
    int eq = ncand;  // candidates whose masked key equals the prefix
    // Most-significant-digit-first radix select, 8-bit digits: per digit, a histogram (this wave's
    // score row, no longer needed, serves as 256 counters) of the candidates that match the prefix,
    // a suffix scan from the largest digit and the digit where the K_i-th largest key lies.
    uint32_t* hist = reinterpret_cast<uint32_t*>(S + rl * a.ld);
#pragma unroll
    for (int k = 0; k < 4; ++k) hist[4 * lane + k] = 0;
    for (int shift = 56; shift >= 0 && eq != need; shift -= 8) {
#pragma unroll
      for (int m = 0; m < SLOTS; ++m)
        if (key[m] != 0 && (key[m] & mask) == prefix) atomicAdd(&hist[(key[m] >> shift) & 255], 1u);
      // lane L holds digits 255 - 4L - k, k = 0..3 (descending)
      uint32_t c[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) c[k] = hist[255 - 4 * lane - k];
      const int tot = int(c[0] + c[1] + c[2] + c[3]);
      const int incl = wave_inclusive_sum(tot);  // candidates with digit >= 252 - 4L
      const uint64_t reach = __ballot(incl >= need);
      const int L = __builtin_ctzll(reach);       // first lane whose range holds the need-th key
      int above = __shfl(incl - tot, L);          // candidates with a larger digit than lane L's
      int d = 255 - 4 * L, cnt = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int ck = __shfl(int(c[k]), L);
        if (cnt == 0 && above + ck >= need) {
          d = 255 - 4 * L - k;
          cnt = ck;
        } else if (cnt == 0) {
          above += ck;
        }
      }
      need -= above;
      eq = cnt;
      prefix |= uint64_t(d) << shift;
      mask |= uint64_t(255) << shift;
#pragma unroll
      for (int k = 0; k < 4; ++k) hist[4 * lane + k] = 0;
    }
    // kept: masked key above the prefix, or equal to it and among the first `need` such (by j);
    // key 0 is never kept (a kept key is at least the K-th largest candidate key, which is > 0)
    int written = 0, ties = 0;
#pragma unroll
    for (int m = 0; m < SLOTS; ++m) {
      const uint64_t km = key[m] & mask;
      const bool c = key[m] != 0;
      const bool tie = c & (km == prefix);
      const uint64_t tb = __ballot(tie);
      const bool sel = (c & (km > prefix)) | (tie & (ties + __popcll(tb & lt_mask) < need));
      ties += __popcll(tb);
      const uint64_t sb = __ballot(sel);
      if (sel) out[written + __popcll(sb & lt_mask)] = lane + 64 * m;
      written += __popcll(sb);
    }
    for (int s = written + lane; s < K; s += 64) out[s] = -1;  // only if row_ptr asks for > n_i
  }
}

// The dynamic-LDS limit of each kernel instantiation is raised once per device (to the largest
// size a row can need), not on every call, so that launches can be captured into a HIP graph.
constexpr int kMaxDevices = 64;

template <int D, int SLOTS, int kRows>
lcsa_status launch(const SelArgs& a, const Geom& g, int bh, hipStream_t s) {
  static std::atomic<uint64_t> raised[kMaxDevices];
  int dev = 0;
  lcsa_status st = hip_status(hipGetDevice(&dev), "lcsa_score_select device");
  if (st != LCSA_OK) return st;
  if (dev < 0 || dev >= kMaxDevices) return fail(LCSA_ERR_UNSUPPORTED, "lcsa_score_select: device %d", dev);
  if (raised[dev].load(std::memory_order_acquire) == 0) {
    const size_t max_lds = size_t(kRows) * (((kMaxCols + 15) / 16) * 16 + kLdsPad) * sizeof(double);
    st = hip_status(hipFuncSetAttribute(reinterpret_cast<const void*>(&score_select_kernel<D, SLOTS, kRows>),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(max_lds)),
                    "lcsa_score_select LDS size");
    if (st != LCSA_OK) return st;
    raised[dev].store(1, std::memory_order_release);
  }
  const size_t lds = size_t(kRows) * a.ld * sizeof(double);
  const int wgs = bh * ((g.nqb + kRows - 1) / kRows);
  score_select_kernel<D, SLOTS, kRows><<<wgs, 64 * kRows, lds, s>>>(a);
  return LCSA_OK;
}

// Rows per workgroup: 16 unless that leaves fewer than 128 workgroups (half the CUs), then 4
// (measured at the 768x1408 chunk, 60 -> 204 workgroups: 21 -> 14 us; at the 1536x2688 chunk,
// with 192 workgroups of 16, the narrow form was slower: it reloads pooled K per 4 rows).
template <int D, int SLOTS>
lcsa_status launch_rows(const SelArgs& a, const Geom& g, int bh, hipStream_t s) {
  if (bh * ((g.nqb + kRowsWide - 1) / kRowsWide) >= 128) return launch<D, SLOTS, kRowsWide>(a, g, bh, s);
  return launch<D, SLOTS, kRowsNarrow>(a, g, bh, s);
}

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
  if (g.nkb > kMaxCols)
    return fail(LCSA_ERR_UNSUPPORTED, "lcsa_score_select: %d key blocks exceed the %d a row can hold",
                g.nkb, kMaxCols);
  int32_t nnz = 0;
  if ((st = lcsa_csr_layout(p, nullptr, nullptr, &nnz, nullptr)) != LCSA_OK) return st;
  SelArgs a{q_pooled, k_pooled, row_ptr, col_idx, scores_dbg, g, nnz, 0, static_cast<double>(p->scale)};
  a.ld = ((g.nkb + 15) / 16) * 16 + kLdsPad;
  if (a.ld < 128) a.ld = 128;  // a row also holds the 256 radix counters of its selection
  const int bh = p->batch * p->heads;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int slots = (g.nkb + 63) / 64;
  if (p->head_dim == 128) {
    if (slots <= 4) st = launch_rows<128, 4>(a, g, bh, s);
    else if (slots <= 8) st = launch_rows<128, 8>(a, g, bh, s);
    else if (slots <= 16) st = launch_rows<128, 16>(a, g, bh, s);
    else st = launch_rows<128, kMaxSlots>(a, g, bh, s);
  } else {
    if (slots <= 4) st = launch_rows<64, 4>(a, g, bh, s);
    else if (slots <= 8) st = launch_rows<64, 8>(a, g, bh, s);
    else if (slots <= 16) st = launch_rows<64, 16>(a, g, bh, s);
    else st = launch_rows<64, kMaxSlots>(a, g, bh, s);
  }
  if (st != LCSA_OK) return st;
  return hip_status(hipGetLastError(), "lcsa_score_select launch");
}
