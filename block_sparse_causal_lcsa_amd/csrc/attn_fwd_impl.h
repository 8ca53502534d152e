// Device code of lcsa_attn_fwd (attn_fwd.hip, attn_fwd_block.hip): exact softmax attention of each
// 128-token query block over the tokens of its kept key blocks (FlashVSR summary, sec. 2.2: full
// attention is applied inside the selected blocks only).
//
// Shared by both kernels below: a wave owns 32 query rows. Scores are computed transposed,
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = key rows from LDS, B = the wave's Q rows held in
// registers), so each lane holds one query row (lane % 32) and half of the 64 or 128 key columns
// and the online softmax needs no cross-lane traffic beyond one swap of row halves. P = exp2(S *
// scale * log2(e) - m) in fp32 is rounded to bf16 and is directly the B operand of O^T += V^T P^T:
// the k-order of the P V MFMA is permuted to match the score layout, and V^T is read from LDS in
// that order. At the end O = O / l (bf16 RNE or fp32) and lse = ln(sum exp(scale q.k)) in fp32.
// Workgroup ids are remapped so that consecutive query blocks of one head run on the same XCD,
// whose L2 then serves the key blocks that neighbouring query blocks share.
//
//  - bf16 (attn_fwd_bf16_kernel): 4 waves per workgroup and query block, two workgroups per CU,
//    K/V tiles loaded directly into LDS; each wave alternates a matrix phase and a vector phase.
//  - fp32 inputs (attn_fwd_kernel): 4 waves per workgroup and query block; tiles are staged through
//    registers, where fp32 is rounded to bf16.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>

#include <type_traits>

#include "lcsa_internal.h"

namespace lcsa {

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;           // [B*Hh, Nq] or null
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int64_t qsb, qsh, qst, ksb, ksh, kst, vsb, vsh, vst, osb, osh, ost;
  Geom g;
  int32_t heads;
  int32_t nnz;
  int32_t nq_tok;       // query tokens per (batch, head)
  int32_t nwg;
  float c;              // scale * log2(e), > 0
  uint32_t k_span, v_span;  // bytes of one (batch, head) slice of K / V
  FastDiv div_bpt, div_wb;  // division by g.bpt and g.Wb
  int32_t nrows;            // (batch, head, query block) rows = B * Hh * nqb
};

// Launches the bf16 kernel for block-granular masks (whole blocks, or partial edge blocks
// when `ragged`; head_dim 64 or 128); defined in attn_fwd_block.hip, which is compiled with a
// different instruction scheduler.
void launch_attn_fwd_bf16_block(const AttnArgs& a, int head_dim, bool ragged, hipStream_t s);

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));


// The running row maximum is only raised when a block's maximum exceeds it by more than this
// (log2 units): P then stays below 2^kLazyMax and O is rescaled only on those rare blocks.
constexpr float kLazyMax = 8.0f;

constexpr int kBN = 128;  // keys per kept block
constexpr int kPadK = 8;  // bf16 elements of padding per LDS row

// Token index (within its tensor) of row r (0..127) of block (tr, hb, wb), tr relative to the
// tensor's first temporal block.
__device__ __forceinline__ int block_token(const Geom& g, int tr, int hb, int wb, int r) {
  return ((kBlkT * tr + (r >> 6)) * g.H + kBlkH * hb + ((r >> 3) & 7)) * g.W + kBlkW * wb + (r & 7);
}

// Query row r (0..127) of block (hb, wb): whether it lies inside the grid, and the row to load in its
// place when it does not (the nearest one inside, so every load stays in the tensor).
__device__ __forceinline__ bool query_row_inside(const Geom& g, int hb, int wb, int r, int* r_load) {
  const int rows = block_rows(g, hb), cols = block_cols(g, wb);
  const int y = (r >> 3) & 7, x = r & 7;
  *r_load = (r & 64) | ((y < rows ? y : rows - 1) << 3) | (x < cols ? x : cols - 1);
  return y < rows && x < cols;
}

// Raw buffer resource over one (batch, head) slice of a token tensor: loads take a 32-bit lane
// offset (VGPR) plus a 32-bit uniform offset (SGPR), so gathers cost no vector ALU work, and any
// access past `bytes` returns zero instead of touching memory. The host guarantees spans < 4 GiB.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr int kBufDword3 = 0x00020000;  // raw 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufDword3);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(__builtin_bit_cast(uint16_t, (__bf16)lo)) |
         (uint32_t(__builtin_bit_cast(uint16_t, (__bf16)hi)) << 16);
}

// Per-thread staging registers for one key block.
template <typename T, int D>
struct Stage {
  static constexpr int KCH = kBN * D / 8 / 256;  // 16-byte bf16 chunks of K per lane
  static constexpr int VGRP = 128 / D;           // 8-key groups per wave instruction set
  static constexpr int VIT = kBN / 8 / 4 / VGRP; // 8-key units per lane
  // K: 8 consecutive d of one key per chunk; V: 2 consecutive d of 8 consecutive keys per unit
  uint32_t k[KCH][4];
  uint32_t v[VIT][8];
};

// Token offset, relative to the block's first token, of key row r (0..127) of a block.
__device__ __forceinline__ int rel_token(const Geom& g, int r) {
  return (r >> 6) * g.H * g.W + ((r >> 3) & 7) * g.W + (r & 7);
}

// Loads key block j into the staging registers. Every address is
//   (uniform block base + wave-uniform row offset) [SGPR] + (loop-invariant per-lane offset) [VGPR].
template <typename T, int D>
__device__ __forceinline__ void stage_load(Stage<T, D>& st, __amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr,
                                           uint32_t kst, uint32_t vst, const Geom& g, int j,
                                           uint32_t k_lane_off, uint32_t v_lane_off) {
  constexpr uint32_t ES = sizeof(T);
  constexpr int CPR = D / 8;        // 8-element chunks per key row
  constexpr int RPI = 256 / CPR;    // key rows per workgroup-wide iteration
  const int tr = j / g.bpt, rem = j - (j / g.bpt) * g.bpt;
  const int hb = rem / g.Wb, wb = rem - (rem / g.Wb) * g.Wb;
  const uint32_t base_tok = uint32_t((kBlkT * tr * g.H + kBlkH * hb) * g.W + kBlkW * wb);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int it = 0; it < Stage<T, D>::KCH; ++it) {
    // rows RPI*it + (RPI/4)*wave + lane/CPR: the lane part stays inside one 8-token row
    const uint32_t soff = (base_tok + uint32_t(rel_token(g, RPI * it + (RPI / 4) * wave))) * kst * ES;
    if constexpr (ES == 2) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(kr, k_lane_off, soff, 0);
      st.k[it][0] = x[0]; st.k[it][1] = x[1]; st.k[it][2] = x[2]; st.k[it][3] = x[3];
    } else {
      const u32x4 x0 = __builtin_amdgcn_raw_buffer_load_b128(kr, k_lane_off, soff, 0);
      const u32x4 x1 = __builtin_amdgcn_raw_buffer_load_b128(kr, k_lane_off + 16, soff, 0);
      st.k[it][0] = pack_bf16x2(__uint_as_float(x0[0]), __uint_as_float(x0[1]));
      st.k[it][1] = pack_bf16x2(__uint_as_float(x0[2]), __uint_as_float(x0[3]));
      st.k[it][2] = pack_bf16x2(__uint_as_float(x1[0]), __uint_as_float(x1[1]));
      st.k[it][3] = pack_bf16x2(__uint_as_float(x1[2]), __uint_as_float(x1[3]));
    }
  }
#pragma unroll
  for (int u = 0; u < Stage<T, D>::VIT; ++u) {
    // unit U = (wave*VIT + u)*VGRP + grp covers V^T columns 8U..8U+7 = keys
    // 16*(U/2) + 4*(U%2) + {0..3, 8..11}; U/2 is wave-uniform, U%2 (only when VGRP = 2) is in the lane offset
    const int G = ((wave * Stage<T, D>::VIT + u) * Stage<T, D>::VGRP) >> 1;
    const int hsel = Stage<T, D>::VGRP == 1 ? (u & 1) : 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 16 * G + 4 * hsel + (e >> 2) * 8 + (e & 3);
      const uint32_t soff = (base_tok + uint32_t(rel_token(g, r))) * vst * ES;
      if constexpr (ES == 2) {
        st.v[u][e] = __builtin_amdgcn_raw_buffer_load_b32(vr, v_lane_off, soff, 0);
      } else {
        const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(vr, v_lane_off, soff, 0);
        st.v[u][e] = pack_bf16x2(__uint_as_float(x[0]), __uint_as_float(x[1]));
      }
    }
  }
}

template <typename T, int D>
__device__ __forceinline__ void stage_store(const Stage<T, D>& st, uint16_t* Ks, uint16_t* Vt) {
  constexpr int KP = D + kPadK, VP = kBN + kPadK;
  constexpr int CPR = D / 8;
  const int t = threadIdx.x;
#pragma unroll
  for (int it = 0; it < Stage<T, D>::KCH; ++it) {
    const int id = t + 256 * it;
    const int r = id / CPR, c = id % CPR;
    *reinterpret_cast<uint4*>(Ks + r * KP + 8 * c) = make_uint4(st.k[it][0], st.k[it][1], st.k[it][2], st.k[it][3]);
  }
  const int wave = t >> 6, lane = t & 63;
  const int dl = lane % (D / 2);
  const int grp = lane / (D / 2);
#pragma unroll
  for (int u = 0; u < Stage<T, D>::VIT; ++u) {
    const int r0 = 8 * ((wave * Stage<T, D>::VIT + u) * Stage<T, D>::VGRP + grp);  // V^T column
    const uint32_t* w = st.v[u];
    // low halves -> row d = 2*dl, high halves -> row 2*dl + 1; 8 consecutive keys each
    const uint4 lo = make_uint4(__builtin_amdgcn_perm(w[1], w[0], 0x05040100u), __builtin_amdgcn_perm(w[3], w[2], 0x05040100u),
                                __builtin_amdgcn_perm(w[5], w[4], 0x05040100u), __builtin_amdgcn_perm(w[7], w[6], 0x05040100u));
    const uint4 hi = make_uint4(__builtin_amdgcn_perm(w[1], w[0], 0x07060302u), __builtin_amdgcn_perm(w[3], w[2], 0x07060302u),
                                __builtin_amdgcn_perm(w[5], w[4], 0x07060302u), __builtin_amdgcn_perm(w[7], w[6], 0x07060302u));
    *reinterpret_cast<uint4*>(Vt + (2 * dl) * VP + r0) = lo;
    *reinterpret_cast<uint4*>(Vt + (2 * dl + 1) * VP + r0) = hi;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(AttnArgs a) {
  constexpr int KP = D + kPadK, VP = kBN + kPadK;
  constexpr int DS = D / 16;  // 16-wide d steps of the QK^T MFMA
  constexpr int DT = D / 32;  // 32-wide d tiles of the output
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kBN * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VP];

  const Geom& g = a.g;
  const int wg = xcd_work_order(blockIdx.x, a.nwg, 1, g.nqb, g.nqb > g.bpt);  // one query block each
  const int bh = wg / g.nqb, i = wg - (wg / g.nqb) * g.nqb;
  const int b = bh / a.heads, h = bh - (bh / a.heads) * a.heads;

  const T* qb = static_cast<const T*>(a.q) + b * a.qsb + h * a.qsh;
  const T* kb = static_cast<const T*>(a.k) + b * a.ksb + h * a.ksh;
  const T* vb = static_cast<const T*>(a.v) + b * a.vsb + h * a.vsh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  const int qtr = i / g.bpt, qrem = i - (i / g.bpt) * g.bpt;
  const int qhb = qrem / g.Wb, qwb = qrem - (qrem / g.Wb) * g.Wb;
  int qrow_ld;
  const bool q_in = query_row_inside(g, qhb, qwb, 32 * wave + l32, &qrow_ld);
  const int qtok = block_token(g, qtr, qhb, qwb, qrow_ld);
  // token-granular window of this lane's query token (rows [lo_h, hi_h], columns [lo_w, hi_w])
  const bool tokwin = token_window(g);
  int lo_h = 0, hi_h = 0, lo_w = 0, hi_w = 0;
  if (tokwin) {
    const bool pres = g.win_mode == kWinTokenPreserving;
    tok_range(pres, kBlkH * qhb + ((qrow_ld >> 3) & 7), g.H, g.wth, &lo_h, &hi_h);
    tok_range(pres, kBlkW * qwb + (qrow_ld & 7), g.W, g.wtw, &lo_w, &hi_w);
  }

  // B operand of S^T = K Q^T: lane holds Q[row l32][16*s + 8*hi + 0..7]
  bf16x8 qf[DS];
  {
    const T* src = qb + int64_t(qtok) * a.qst + 8 * hi;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      if constexpr (sizeof(T) == 2) {
        qf[s] = *reinterpret_cast<const bf16x8*>(src + 16 * s);
      } else {
        const float4 x0 = *reinterpret_cast<const float4*>(src + 16 * s);
        const float4 x1 = *reinterpret_cast<const float4*>(src + 16 * s + 4);
        qf[s] = bf16x8{(__bf16)x0.x, (__bf16)x0.y, (__bf16)x0.z, (__bf16)x0.w,
                       (__bf16)x1.x, (__bf16)x1.y, (__bf16)x1.z, (__bf16)x1.w};
      }
    }
  }

  const uint32_t kst32 = static_cast<uint32_t>(a.kst), vst32 = static_cast<uint32_t>(a.vst);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kb, a.k_span), vrs = make_rsrc(vb, a.v_span);
  // per-lane parts of the staging addresses (see stage_load)
  const uint32_t k_lane_off = ((lane / (D / 8)) * kst32 + 8 * (lane % (D / 8))) * uint32_t(sizeof(T));
  const uint32_t v_lane_off = (4 * (lane / (D / 2)) * vst32 + 2 * (lane % (D / 2))) * uint32_t(sizeof(T));
  const int beg = a.row_ptr[i], nsel = a.row_ptr[i + 1] - beg;
  const int32_t* sel = a.col_idx + int64_t(bh) * a.nnz + beg;

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  Stage<T, D> st;
  // entries outside [0, nkb) are replaced by block 0 and contribute exactly zero (see neg_m)
  int jn = nsel > 0 ? sel[0] : 0;
  bool ok_next = jn >= 0 && jn < g.nkb;
  stage_load<T, D>(st, krs, vrs, kst32, vst32, g, ok_next ? jn : 0, k_lane_off, v_lane_off);

  for (int n = 0; n < nsel; ++n) {
    const bool ok = ok_next;
    const int jcur = ok ? jn : 0;
    __syncthreads();  // every wave is done reading the previous block
    stage_store<T, D>(st, Ks, Vt);
    __syncthreads();
    // next block (the last iteration re-reads the current one, which is in L2, to keep the loop
    // free of branches around the staging registers)
    jn = n + 1 < nsel ? sel[n + 1] : jcur;
    ok_next = jn >= 0 && jn < g.nkb;

    // S^T tiles: 4 x (32 keys x 32 queries); the four accumulators are independent chains
    f32x16 sacc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) sacc[kt] = f32x16{};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (kt * 32 + l32) * KP + 8 * hi + 16 * s);
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[kt], 0, 0, 0);
      }
    }
    {
      const int rem = jcur % g.bpt, hbk = rem / g.Wb, wbk = rem % g.Wb;
      if (tokwin) {
        // keys outside this query token's window (which also excludes tokens past the grid edge)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
          mask_window_tile(sacc[kt], kt & 1, hi, kBlkH * hbk, kBlkW * wbk, lo_h, hi_h, lo_w, hi_w);
      } else {
        // keys outside the grid in a partial block (last block row / column)
        const int rows = block_rows(g, hbk), cols = block_cols(g, wbk);
        if (rows < kBlkH || cols < kBlkW) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) mask_partial_tile(sacc[kt], kt & 1, hi, rows, cols);
        }
      }
    }
    // online softmax in the log2 domain; this lane holds 64 of the row's 128 raw scores
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kt][v]);
    mx = ok ? fmaxf(mx, __shfl_xor(mx, 32)) * a.c : -INFINITY;  // c > 0, so max(c s) = c max(s)
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyMax)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
    }
    // a skipped entry, or a row that has seen no key yet, gives P = exp2(-inf) = 0
    const float neg_m = ok && m_run != -INFINITY ? -m_run : -INFINITY;
    float ls = 0.f;
    bf16x8 pf[4][2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][8 * h2 + e], a.c, neg_m));
          ls += pv;
          pf[kt][h2][e] = (__bf16)pv;
        }
    l_run += ls;

    // the next block's loads overlap the PV MFMAs (issued here to keep fewer registers live)
    stage_load<T, D>(st, krs, vrs, kst32, vst32, g, ok_next ? jn : 0, k_lane_off, v_lane_off);

    // O^T += V^T P^T. MFMA k-slot 8*hi + e of step (kt, h2) is key kt*32 + 16*h2 + 8*(e/4) + 4*hi + e%4,
    // where the score layout put P; V^T stores those 8 keys contiguously (columns 16*(2kt+h2) + 8*hi).
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(Vt + (dt * 32 + l32) * VP + 16 * (2 * kt + h2) + 8 * hi);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[kt][h2], oacc[dt], 0, 0, 0);
        }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (!q_in) return;  // a query row outside the grid (partial block) has no output
  T* ob = static_cast<T*>(a.o) + b * a.osb + h * a.osh + int64_t(qtok) * a.ost;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      // items 4*g4..4*g4+3 are d = dt*32 + 8*g4 + 4*hi + 0..3
      const int d0 = dt * 32 + 8 * g4 + 4 * hi;
      const float o0 = oacc[dt][4 * g4] * inv, o1 = oacc[dt][4 * g4 + 1] * inv;
      const float o2 = oacc[dt][4 * g4 + 2] * inv, o3 = oacc[dt][4 * g4 + 3] * inv;
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint2*>(ob + d0) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
      } else {
        *reinterpret_cast<float4*>(ob + d0) = make_float4(o0, o1, o2, o3);
      }
    }
  if (a.lse && hi == 0) {
    const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    a.lse[int64_t(bh) * a.nq_tok + qtok] = lse;
  }
}


// ------------------------------------------------------------------------------------------------
// bf16 inputs: each kept key block is processed as two 64-key sub-blocks (its two latent frames).
// Sub-block tiles of K and V go straight from memory into LDS with buffer loads (no registers, no
// LDS stores).
//   K tile: [key][d], 16-byte chunk c of key row r at chunk position c ^ (r mod CPR): the QK^T
//           fragment reads (16 lanes on 16 consecutive rows, one chunk) hit distinct banks.
//   V tile: [key][d], chunk c of row r at c ^ vswz(r); the PV operand (V^T) is read with
//           ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i%4 of the 8-byte
//           pieces addressed by lanes 4k + (i%16)/4, k = 0..3, so pointing lane j at key row
//           K0 + j/4, columns d0 + 4(j%4) delivers V[K0 + k][d0 + i%16] to lane i: four consecutive
//           keys of one head-dim column, exactly an MFMA A-operand half.
constexpr int kSub = 64;  // keys per sub-block
// Bound on a lane's sum of 32 unnormalised probabilities before the running maximum is refreshed:
// every P stays below 2^16, far from overflowing the fp32 accumulators for finite inputs.
constexpr float kSumMax = 65536.0f;

template <int D>
struct Tile {
  static constexpr int CPR = D / 8;               // 16-byte chunks per key row
  static constexpr int LOADS = kSub * CPR / 256;  // 16-byte loads per lane per tile
  static constexpr int ELEMS = kSub * D;          // bf16 elements per tile
};

template <int D>
__device__ __forceinline__ int vswz(int r) {
  return Tile<D>::CPR >= 16 ? 4 * (r & 3) : 4 * (r & 1);
}

// Issues the loads of one sub-block tile (K or V) of `ELEMS` bf16 into LDS at `tile`.
// Rows r of the tile are tokens (r/8)*W + r%8 after `base_tok` (one latent frame of the block).
// Load `it` (0 .. LOADS-1) of this wave's share of a tile: 64 lanes x 16 bytes.
template <int D, bool IS_V>
__device__ __forceinline__ void issue_tile_part(__amdgpu_buffer_rsrc_t rs, uint16_t* tile, uint32_t tst, uint32_t base_tok,
                                                int W, int wave, int lane, int it) {
  constexpr int CPR = Tile<D>::CPR;
  const int slot0 = (wave * Tile<D>::LOADS + it) * 64;  // first 16-byte slot of this wave instruction
  const int r0 = slot0 / CPR;                           // first row (a multiple of 64 / CPR)
  const int r = r0 + lane / CPR;                        // stays inside one 8-token row
  const int pos = lane % CPR;
  const int c = pos ^ (IS_V ? vswz<D>(r) : (r & (CPR - 1)));
  const uint32_t soff = (base_tok + uint32_t((r0 / 8) * W + (r0 % 8))) * tst * 2u;
  const uint32_t voff = (uint32_t(lane / CPR) * tst + 8u * uint32_t(c)) * 2u;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rs, (__attribute__((address_space(3))) void*)(tile + slot0 * 8), 16, voff, soff, 0, 0);
}

template <int D, bool IS_V>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t rs, uint16_t* tile, uint32_t tst, uint32_t base_tok,
                                           int W, int wave, int lane) {
#pragma unroll
  for (int it = 0; it < Tile<D>::LOADS; ++it) issue_tile_part<D, IS_V>(rs, tile, tst, base_tok, W, wave, lane, it);
}

// Largest raw score of this lane's query row over the tile (both lane halves hold halves of a row).
__device__ __forceinline__ float tile_rowmax(const f32x16 (&s)[2]) {
  float m0 = s[0][0], m1 = s[1][0];
#pragma unroll
  for (int v = 1; v < 16; ++v) {
    m0 = fmaxf(m0, s[0][v]);
    m1 = fmaxf(m1, s[1][v]);
  }
  const float mx = fmaxf(m0, m1);
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
  return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
}

// ------------------------------------------------------------------------------------------------
// Phase schedule (bf16). A workgroup of 4 waves owns one query block, and two workgroups share a CU,
// so each SIMD runs one wave of each. A wave alternates a matrix phase (P V of the previous sub-block
// and Q K^T of the current one: 32 MFMAs) and a vector phase (exponentials, bf16 packing and row
// sums of the current sub-block); phases end at workgroup barriers. The two waves of a SIMD are not
// locked to each other: vector work of one wave does not overlap the other's MFMAs on this hardware
// (measured), so a ping-pong lock of two query blocks (one wave in each phase at every moment) only
// adds barrier waits.
// M(m) reads K(m) and V(m-1) from LDS; the vector phase V(m) issues the direct-to-LDS loads of K(m+2)
// and V(m+1) (their buffers were last read in M(m)) and, at its end, waits for the loads of K(m+1)
// and V(m), issued one vector phase earlier, which M(m+1) reads.
typedef const __attribute__((address_space(4))) int32_t const_i32;

// Barrier between phases without a memory fence: the direct-to-LDS loads in flight stay in flight.
// Every LDS read this wave issued has completed (lgkmcnt(0)).
// Nothing is scheduled across it, so every phase keeps its own instructions.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Waits until at most n (0, 1 or 2) tiles' worth of this lane's direct-to-LDS loads are in flight.
template <int LOADS>
__device__ __forceinline__ void wait_tiles(int n) {
  if (n >= 2) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LOADS) : "memory");
  } else if (n == 1) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }
}

// MASK: kMaskNone for whole blocks and a block-granular window (no token mask at all);
// kMaskRagged when the grid is not a multiple of 8 (partial edge blocks: masked keys, query rows
// without output); kMaskWindow for a token-granular window (per-token masks in the blocks that are
// not wholly inside every query token's window; also covers partial blocks).
constexpr int kMaskNone = 0, kMaskRagged = 1, kMaskWindow = 2;

template <int D, int MASK>
__device__ __forceinline__ void attn_group(const AttnArgs& a, int qblk, int row_start, int nsel, int lwave,
                                         uint16_t* kb0, uint16_t* kb1, uint16_t* vb0, uint16_t* vb1) {
  constexpr int DS = D / 16;
  constexpr int DT = D / 32;
  constexpr int CPR = Tile<D>::CPR;
  constexpr int LOADS = Tile<D>::LOADS;
  const Geom& g = a.g;
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int t = 2 * nsel;

  const int bh = qblk / g.nqb, i = qblk - bh * g.nqb;
  const int b = bh / a.heads, h = bh - (bh / a.heads) * a.heads;
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + b * a.qsb + h * a.qsh;
  const uint16_t* kbp = static_cast<const uint16_t*>(a.k) + b * a.ksb + h * a.ksh;
  const uint16_t* vbp = static_cast<const uint16_t*>(a.v) + b * a.vsb + h * a.vsh;
  const int qtr = i / g.bpt, qrem = i - (i / g.bpt) * g.bpt;
  const int qhb = qrem / g.Wb, qwb = qrem - (qrem / g.Wb) * g.Wb;
  int qrow_ld = 32 * lwave + l32;
  const bool q_in = MASK != kMaskNone ? query_row_inside(g, qhb, qwb, 32 * lwave + l32, &qrow_ld) : true;
  const int qtok = block_token(g, qtr, qhb, qwb, qrow_ld);
  // token-granular window: this lane's query token sees rows [lo_h, hi_h], columns [lo_w, hi_w]; a key
  // block inside [lo_max, hi_min] on both axes is seen whole by every token of the query block
  int lo_h = 0, hi_h = 0, lo_w = 0, hi_w = 0, lo_max_h = 0, hi_min_h = 0, lo_max_w = 0, hi_min_w = 0;
  if constexpr (MASK == kMaskWindow) {
    const bool pres = g.win_mode == kWinTokenPreserving;
    tok_range(pres, kBlkH * qhb + ((qrow_ld >> 3) & 7), g.H, g.wth, &lo_h, &hi_h);
    tok_range(pres, kBlkW * qwb + (qrow_ld & 7), g.W, g.wtw, &lo_w, &hi_w);
    int t0, t1;
    tok_range(pres, kBlkH * qhb + block_rows(g, qhb) - 1, g.H, g.wth, &lo_max_h, &t1);
    tok_range(pres, kBlkH * qhb, g.H, g.wth, &t0, &hi_min_h);
    tok_range(pres, kBlkW * qwb + block_cols(g, qwb) - 1, g.W, g.wtw, &lo_max_w, &t1);
    tok_range(pres, kBlkW * qwb, g.W, g.wtw, &t0, &hi_min_w);
  }

  bf16x8 qf[DS];
  {
    const uint16_t* src = qb + int64_t(qtok) * a.qst + 8 * hi;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(src + 16 * s);
  }

  const uint32_t kst = static_cast<uint32_t>(a.kst), vst = static_cast<uint32_t>(a.vst);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbp, a.k_span), vrs = make_rsrc(vbp, a.v_span);
  // the column list is read-only for the whole launch: read it through the scalar cache (uniform
  // scalar loads, which leave the vector-memory counter to the tile loads)
  const const_i32* sel = (const const_i32*)(a.col_idx) + int64_t(bh) * a.nnz + row_start;
  const uint32_t hw = uint32_t(g.H) * uint32_t(g.W);
  // first token of kept block j; ok: j is a block; lim: 16 * rows + cols inside the grid (136: full)
  auto block_base = [&](int j, bool& ok, int& lim) -> uint32_t {
    ok = j >= 0 && j < g.nkb;
    const uint32_t ju = ok ? uint32_t(j) : 0u;
    const uint32_t tr = fast_div(ju, a.div_bpt), rem = ju - tr * uint32_t(g.bpt);
    const uint32_t hb = fast_div(rem, a.div_wb), wb = rem - hb * uint32_t(g.Wb);
    if constexpr (MASK == kMaskRagged) lim = 16 * block_rows(g, int(hb)) + block_cols(g, int(wb));
    if constexpr (MASK == kMaskWindow) {
      const int h0 = kBlkH * int(hb), w0 = kBlkW * int(wb);
      const bool whole = h0 >= lo_max_h && h0 + kBlkH - 1 <= hi_min_h && w0 >= lo_max_w && w0 + kBlkW - 1 <= hi_min_w;
      lim = whole ? -1 : ((int(hb) << 16) | int(wb));
    }
    return (kBlkT * tr * uint32_t(g.H) + kBlkH * hb) * uint32_t(g.W) + kBlkW * wb;
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const int kx = l32 & (CPR - 1);
  const int jj = lane & 15;
  const int vrow = 4 * hi + jj / 4;
  const int vcol = (lane & 16) + 4 * (jj & 3);

  // block n = current (ok_c, base_c), n + 1 (ok_n, base_n), entry of n + 2 (j_pref)
  bool ok_c = false, ok_n = false;
  int lim_c = 136, lim_n = 136;
  uint32_t base_c = 0, base_n = 0;
  int j_pref = 0;
  if (t > 0) {
    base_c = block_base(sel[0], ok_c, lim_c);
    if (nsel > 1) base_n = block_base(sel[1], ok_n, lim_n);
    if (nsel > 2) j_pref = sel[2];
    issue_tile<D, false>(krs, kb0, kst, base_c, g.W, lwave, lane);
    issue_tile<D, false>(krs, kb1, kst, base_c + hw, g.W, lwave, lane);
    issue_tile<D, true>(vrs, vb0, vst, base_c, g.W, lwave, lane);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  phase_barrier();

  f32x16 S[2];
  bf16x8 pf[2][2];

  // matrix phase: O += V^T P^T of the previous sub-block (tile Vp), S = K Q^T of the current (tile Kc).
  // Every MFMA takes one 16-byte operand fragment
  // from LDS, read kLook MFMAs ahead so the LDS latency hides behind the matrix core.
  auto mphase = [&](const uint16_t* Vp, const uint16_t* Kc, auto pv_tag, auto qk_tag) __attribute__((always_inline)) {
    constexpr bool do_pv = decltype(pv_tag)::value, do_qk = decltype(qk_tag)::value;
    constexpr int NQ = do_qk ? 2 * DS : 0;  // Q K^T MFMAs: (d step st, key tile kt)
    constexpr int NP = do_pv ? 4 * DT : 0;  // P V MFMAs: (key tile kt, half h2, d tile dt)
    constexpr int NOPS = NQ + NP;
    constexpr int kLook = 4;
    // op j: with both products, even j are Q K^T ops and odd j are P V ops
    auto is_qk = [](int j) { return NP == 0 ? true : (NQ == 0 ? false : (j % 2 == 0)); };
    auto sub = [](int j) { return (NP == 0 || NQ == 0) ? j : j / 2; };
    auto load = [&](int j) -> bf16x8 {
      if (is_qk(j)) {
        const int q = sub(j), st = q >> 1, kt = q & 1;
        return *reinterpret_cast<const bf16x8*>(Kc + (kt * 32 + l32) * D + (((2 * st + hi) ^ kx) * 8));
      }
      const int q = sub(j), kt = q / (2 * DT), h2 = (q / DT) & 1, dt = q % DT;
      v4i16 part[2];
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const int row = kt * 32 + 16 * h2 + 8 * e2 + vrow;
        const int col = dt * 32 + vcol;
        const uint16_t* p = Vp + row * D + ((((col >> 3) ^ vswz<D>(row)) << 3) | (col & 7));
        part[e2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
      }
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
    };
    if constexpr (do_qk) {
      S[0] = f32x16{};
      S[1] = f32x16{};
    }
    bf16x8 fr[kLook];
#pragma unroll
    for (int j = 0; j < kLook && j < NOPS; ++j) fr[j] = load(j);
#pragma unroll
    for (int j = 0; j < NOPS; ++j) {
      const bf16x8 f = fr[j % kLook];
      if (j + kLook < NOPS) fr[j % kLook] = load(j + kLook);
      if (is_qk(j)) {
        const int q = sub(j), st = q >> 1, kt = q & 1;
        S[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, qf[st], S[kt], 0, 0, 0);
      } else {
        const int q = sub(j), kt = q / (2 * DT), h2 = (q / DT) & 1, dt = q % DT;
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, pf[kt][h2], oacc[dt], 0, 0, 0);
      }
    }
  };

  // vector phase: online softmax of the current sub-block (scores S, block validity ok). The running
  // maximum is only refreshed when the exponentials overflow a bound: P = 2^(c s - m_run) is computed
  // first, and when any lane's partial sum exceeds kSumMax (or is not finite, as on the first block,
  // where m_run = -inf) the row maximum is taken, O and l are rescaled and P is recomputed.
  auto exps = [&](float neg_m) __attribute__((always_inline)) -> float {
    float x[2][16];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) x[kt][v] = __builtin_fmaf(S[kt][v], a.c, neg_m);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) x[kt][v] = __builtin_amdgcn_exp2f(x[kt][v]);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[kt][h2][e] = (__bf16)x[kt][8 * h2 + e];
    // row sum of the fp32 probabilities, before their rounding to bf16: the denominator (and lse)
    // stay exact to fp32 even when one rounded probability carries most of a row's mass
    // (the chains start at the first four values: the same sums as from 0, without four adds)
    float acc[4] = {x[0][0], x[0][1], x[0][2], x[0][3]};
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = kt == 0 ? 4 : 0; v < 16; ++v) acc[v & 3] += x[kt][v];
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
  };
  auto vphase = [&](bool ok, int lim) __attribute__((always_inline)) {
    if constexpr (MASK == kMaskRagged) {
      if (lim != 16 * kBlkH + kBlkW) {  // partial block at the grid edge (uniform branch)
        mask_partial_tile(S[0], 0, hi, lim >> 4, lim & 15);
        mask_partial_tile(S[1], 1, hi, lim >> 4, lim & 15);
      }
    }
    if constexpr (MASK == kMaskWindow) {
      if (lim >= 0) {  // a block not seen whole by every query token (uniform branch)
        const int h0 = kBlkH * (lim >> 16), w0 = kBlkW * (lim & 0xffff);
        mask_window_tile(S[0], 0, hi, h0, w0, lo_h, hi_h, lo_w, hi_w);
        mask_window_tile(S[1], 1, hi, h0, w0, lo_h, hi_h, lo_w, hi_w);
      }
      // a row may see no key yet: its running maximum stays -inf and its probabilities 0, and every
      // sub-block refreshes it until it sees one
      float ls = exps(ok && m_run != -INFINITY ? -m_run : -INFINITY);
      if (__builtin_amdgcn_ballot_w64(!(ls <= kSumMax) || (ok && m_run == -INFINITY))) {
        const float mxs = ok ? tile_rowmax(S) * a.c : -INFINITY;
        const float m_new = fmaxf(m_run, mxs);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
        ls = exps(ok && m_run != -INFINITY ? -m_run : -INFINITY);
      }
      l_run += ls;
    } else {
      float ls = exps(ok ? -m_run : -INFINITY);
      if (__builtin_amdgcn_ballot_w64(!(ls <= kSumMax))) {
        const float mxs = ok ? tile_rowmax(S) * a.c : -INFINITY;
        const float m_new = fmaxf(m_run, mxs);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 while m_run = -inf
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
        ls = exps(ok ? -m_run : -INFINITY);
      }
      l_run += ls;
    }
  };

  using Yes = std::integral_constant<bool, true>;
  using No = std::integral_constant<bool, false>;
  // one kept block n: sub-blocks m = 2n (frame 0) and m = 2n + 1 (frame 1); MORE: block n + 1 exists
  auto block_iter = [&](int n, auto more_tag) __attribute__((always_inline)) {
    constexpr bool MORE = decltype(more_tag)::value;
    const int jn = n + 3 < nsel ? sel[n + 3] : 0;  // entry of block n + 3, needed two blocks later
    // ---- vector phase of m = 2n
    if constexpr (MORE) issue_tile<D, false>(krs, kb0, kst, base_n, g.W, lwave, lane);  // K(n+1, 0)
    issue_tile<D, true>(vrs, vb1, vst, base_c + hw, g.W, lwave, lane);                 // V(n, 1)
    vphase(ok_c, lim_c);
    wait_tiles<LOADS>(MORE ? 2 : 1);  // K(n, 1) and V(n, 0) have landed
    phase_barrier();
    mphase(vb0, kb1, Yes{}, Yes{});  // P V(n, 0); S = K(n, 1) Q^T
    phase_barrier();
    // ---- vector phase of m = 2n + 1
    if constexpr (MORE) {
      issue_tile<D, false>(krs, kb1, kst, base_n + hw, g.W, lwave, lane);  // K(n+1, 1)
      issue_tile<D, true>(vrs, vb0, vst, base_n, g.W, lwave, lane);        // V(n+1, 0)
    }
    vphase(ok_c, lim_c);
    wait_tiles<LOADS>(MORE ? 2 : 0);  // K(n+1, 0) and V(n, 1) have landed
    phase_barrier();
    if constexpr (MORE) {
      mphase(vb1, kb0, Yes{}, Yes{});  // P V(n, 1); S = K(n+1, 0) Q^T
    } else {
      mphase(vb1, kb0, Yes{}, No{});
    }
    phase_barrier();
    ok_c = ok_n;
    lim_c = lim_n;
    base_c = base_n;
    base_n = block_base(j_pref, ok_n, lim_n);
    j_pref = jn;
  };

  if (t > 0) {
    mphase(vb1, kb0, No{}, Yes{});  // M(0): S = K(0, 0) Q^T
    phase_barrier();
    for (int n = 0; n + 1 < nsel; ++n) block_iter(n, Yes{});
    block_iter(nsel - 1, No{});
  }

  if (!q_in) return;  // a query row outside the grid (partial block) has no output
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* ob = static_cast<uint16_t*>(a.o) + b * a.osb + h * a.osh + int64_t(qtok) * a.ost;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = dt * 32 + 8 * g4 + 4 * hi;
      *reinterpret_cast<uint2*>(ob + d0) =
          make_uint2(pack_bf16x2(oacc[dt][4 * g4] * inv, oacc[dt][4 * g4 + 1] * inv),
                     pack_bf16x2(oacc[dt][4 * g4 + 2] * inv, oacc[dt][4 * g4 + 3] * inv));
    }
  if (a.lse && hi == 0) {
    const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
    a.lse[int64_t(bh) * a.nq_tok + qtok] = lse;
  }
}

template <int D, int MASK>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(AttnArgs a) {
  constexpr int TE = Tile<D>::ELEMS;
  __shared__ __attribute__((aligned(16))) uint16_t k0[TE];
  __shared__ __attribute__((aligned(16))) uint16_t k1[TE];
  __shared__ __attribute__((aligned(16))) uint16_t v0[TE];
  __shared__ __attribute__((aligned(16))) uint16_t v1[TE];
  const int qblk = xcd_work_order(blockIdx.x, a.nwg, 1, a.g.nqb, a.g.nqb > a.g.bpt);  // one query block each
  const const_i32* rp = (const const_i32*)(a.row_ptr);
  const int i = qblk % a.g.nqb;
  const int r0 = rp[i], n = rp[i + 1] - r0;
  const int lwave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  attn_group<D, MASK>(a, qblk, r0, n, lwave, k0, k1, v0, v1);
}

}  // namespace
}  // namespace lcsa
