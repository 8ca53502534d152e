// lcsa_attn_fwd: exact softmax attention of each 128-token query block over the tokens of its kept
// key blocks (FlashVSR summary, sec. 2.2: full attention is applied inside the selected blocks only).
//
// One workgroup (4 waves, 256 lanes) per (batch, head, query block); wave w owns query rows
// 32w..32w+31 of the block. For every kept key block j (128 tokens):
//   - K_j is staged in LDS row-major [key][d] and V_j transposed [d][key] (bf16), from registers that
//     were loaded from HBM/L2 while the previous block was being computed;
//   - S^T = K_j Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = the wave's Q rows held in
//     registers). In the result each lane holds one query row (lane % 32) and half of the key
//     columns, so the online softmax needs one cross-lane max per block and no other exchange;
//   - the scores become P = exp2(S * scale * log2(e) - m) in fp32 (running max m, running sum l),
//     P is rounded to bf16 and used directly as the B operand of O^T += V_j^T P^T: the k-order of
//     the PV MFMA is permuted to match the score layout, and V^T is read from LDS in that order.
// At the end O = O / l (bf16 RNE or fp32) and lse = ln(sum exp(scale q.k)) in fp32.
// Workgroup ids are remapped so that consecutive query blocks of one head run on the same XCD,
// whose L2 then serves the key blocks that neighbouring query blocks share.
#include <hip/hip_runtime.h>

#include <math.h>

#include "lcsa_internal.h"

namespace lcsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

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
};

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
  // XCD-aware order: hardware deals workgroup n to XCD n % 8; give each XCD a contiguous range
  int wg = blockIdx.x;
  const int n8 = (a.nwg / 8) * 8;
  if (wg < n8) wg = (wg % 8) * (a.nwg / 8) + wg / 8;
  const int bh = wg / g.nqb, i = wg - (wg / g.nqb) * g.nqb;
  const int b = bh / a.heads, h = bh - (bh / a.heads) * a.heads;

  const T* qb = static_cast<const T*>(a.q) + b * a.qsb + h * a.qsh;
  const T* kb = static_cast<const T*>(a.k) + b * a.ksb + h * a.ksh;
  const T* vb = static_cast<const T*>(a.v) + b * a.vsb + h * a.vsh;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  const int qtr = i / g.bpt, qrem = i - (i / g.bpt) * g.bpt;
  const int qhb = qrem / g.Wb, qwb = qrem - (qrem / g.Wb) * g.Wb;
  const int qtok = block_token(g, qtr, qhb, qwb, 32 * wave + l32);

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
    // online softmax in the log2 domain; this lane holds 64 of the row's 128 raw scores
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kt][v]);
    mx = ok ? fmaxf(mx, __shfl_xor(mx, 32)) * a.c : -INFINITY;  // c > 0, so max(c s) = c max(s)
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyMax)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
    }
    const float neg_m = ok ? -m_run : -INFINITY;  // a skipped entry gives P = exp2(-inf) = 0
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
// LDS stores), double-buffered, so one workgroup barrier per sub-block both publishes the tile that
// just landed and frees the buffer the next loads go to.
//   K tile: [key][d], 16-byte chunk c of key row r at chunk position c ^ (r mod CPR): the QK^T
//           fragment reads (16 lanes on 16 consecutive rows, one chunk) hit distinct banks.
//   V tile: [key][d], chunk c of row r at c ^ vswz(r); the PV operand (V^T) is read with
//           ds_read_b64_tr_b16: in each 16-lane group, lane i receives element i%4 of the 8-byte
//           pieces addressed by lanes 4k + (i%16)/4, k = 0..3, so pointing lane j at key row
//           K0 + j/4, columns d0 + 4(j%4) delivers V[K0 + k][d0 + i%16] to lane i: four consecutive
//           keys of one head-dim column, exactly an MFMA A-operand half.
constexpr int kSub = 64;  // keys per sub-block

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
template <int D, bool IS_V>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t rs, uint16_t* tile, uint32_t tst, uint32_t base_tok,
                                           int W, int wave, int lane) {
  constexpr int CPR = Tile<D>::CPR;
#pragma unroll
  for (int it = 0; it < Tile<D>::LOADS; ++it) {
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
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_direct_kernel(AttnArgs a) {
  constexpr int DS = D / 16;  // 16-wide d steps of the QK^T MFMA
  constexpr int DT = D / 32;  // 32-wide d tiles of the output
  constexpr int CPR = Tile<D>::CPR;
  constexpr int TE = Tile<D>::ELEMS;
  // two buffers, each [K | V]; separate arrays so the compiler can tell the buffer being read from
  // the one the in-flight loads write
  __shared__ __attribute__((aligned(16))) uint16_t buf0[2 * TE];
  __shared__ __attribute__((aligned(16))) uint16_t buf1[2 * TE];

  const Geom& g = a.g;
  int wg = blockIdx.x;
  const int n8 = (a.nwg / 8) * 8;
  if (wg < n8) wg = (wg % 8) * (a.nwg / 8) + wg / 8;
  const int bh = wg / g.nqb, i = wg - (wg / g.nqb) * g.nqb;
  const int b = bh / a.heads, h = bh - (bh / a.heads) * a.heads;

  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + b * a.qsb + h * a.qsh;
  const uint16_t* kb = static_cast<const uint16_t*>(a.k) + b * a.ksb + h * a.ksh;
  const uint16_t* vb = static_cast<const uint16_t*>(a.v) + b * a.vsb + h * a.vsh;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  const int qtr = i / g.bpt, qrem = i - (i / g.bpt) * g.bpt;
  const int qhb = qrem / g.Wb, qwb = qrem - (qrem / g.Wb) * g.Wb;
  const int qtok = block_token(g, qtr, qhb, qwb, 32 * wave + l32);

  // B operand of S^T = K Q^T: lane holds Q[row l32][16*s + 8*hi + 0..7]
  bf16x8 qf[DS];
  {
    const uint16_t* src = qb + int64_t(qtok) * a.qst + 8 * hi;
#pragma unroll
    for (int s = 0; s < DS; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(src + 16 * s);
  }

  const uint32_t kst = static_cast<uint32_t>(a.kst), vst = static_cast<uint32_t>(a.vst);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kb, a.k_span), vrs = make_rsrc(vb, a.v_span);
  const int beg = a.row_ptr[i], nsel = a.row_ptr[i + 1] - beg;
  const int32_t* sel = a.col_idx + int64_t(bh) * a.nnz + beg;
  const int total = 2 * nsel;
  const uint32_t hw = uint32_t(g.H) * uint32_t(g.W);

  // first token of sub-block m (block sel[m/2], latent frame m%2); entries outside [0, nkb) use
  // block 0 and are masked out of the softmax
  auto sub_base = [&](int m, bool& ok) -> uint32_t {
    int j = sel[m >> 1];
    ok = j >= 0 && j < g.nkb;
    j = ok ? j : 0;
    const int tr = j / g.bpt, rem = j - (j / g.bpt) * g.bpt;
    const int hb = rem / g.Wb, wb = rem - (rem / g.Wb) * g.Wb;
    return uint32_t((kBlkT * tr * g.H + kBlkH * hb) * g.W + kBlkW * wb) + uint32_t(m & 1) * hw;
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  // lane parts of the LDS fragment addresses
  const int kx = l32 & (CPR - 1);  // K swizzle of rows kt*32 + l32
  const int jj = lane & 15;
  const int vrow = 4 * hi + jj / 4;                 // V^T read: row offset inside a 16-key group
  const int vcol = (lane & 16) + 4 * (jj & 3);      // and column offset inside a 32-wide d tile

  bool ok_next = true;
  uint32_t base_next = total > 0 ? sub_base(0, ok_next) : 0;
  if (total > 0) {
    issue_tile<D, false>(krs, buf0, kst, base_next, g.W, wave, lane);
    issue_tile<D, true>(vrs, buf0 + TE, vst, base_next, g.W, wave, lane);
  }

  // one sub-block: wait for its tile in `cur`, start loading the next one into `nxt`, compute
  auto step = [&](int m, const uint16_t* cur, uint16_t* nxt) __attribute__((always_inline)) {
    const bool ok = ok_next;
    const uint16_t* Kt = cur;
    const uint16_t* Vt = cur + TE;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this lane's tile loads have landed
    __syncthreads();  // every lane's have; and every wave is done with the other buffer
    if (m + 1 < total) {
      base_next = sub_base(m + 1, ok_next);
      uint16_t* nk = nxt;
      issue_tile<D, false>(krs, nk, kst, base_next, g.W, wave, lane);
      issue_tile<D, true>(vrs, nk + TE, vst, base_next, g.W, wave, lane);
    }

    // S^T: 2 x (32 keys x 32 queries)
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int s = 0; s < DS; ++s) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Kt + (kt * 32 + l32) * D + (((2 * s + hi) ^ kx) * 8));
        sacc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[kt], 0, 0, 0);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kt][v]);
    mx = ok ? fmaxf(mx, __shfl_xor(mx, 32)) * a.c : -INFINITY;  // c > 0
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyMax)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
    }
    const float neg_m = ok ? -m_run : -INFINITY;
    float ls = 0.f;
    bf16x8 pf[2][2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][8 * h2 + e], a.c, neg_m));
          ls += pv;
          pf[kt][h2][e] = (__bf16)pv;
        }
    l_run += ls;

    // O^T += V^T P^T; k-slot 8*hi + e of step (kt, h2) is key kt*32 + 16*h2 + 8*(e/4) + 4*hi + e%4
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          v4i16 part[2];
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            const int row = kt * 32 + 16 * h2 + 8 * e2 + vrow;
            const int col = dt * 32 + vcol;
            const uint16_t* p = Vt + row * D + ((((col >> 3) ^ vswz<D>(row)) << 3) | (col & 7));
            part[e2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
          }
          const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[kt][h2], oacc[dt], 0, 0, 0);
        }
  };
  for (int m = 0; m < total; m += 2) {
    step(m, buf0, buf1);
    if (m + 1 < total) step(m + 1, buf1, buf0);
  }

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

}  // namespace
}  // namespace lcsa

using namespace lcsa;

extern "C" lcsa_status lcsa_attn_fwd(const lcsa_problem* p, const void* q, lcsa_strides qs, const void* k,
                                     lcsa_strides ks, const void* v, lcsa_strides vs, const int32_t* row_ptr,
                                     const int32_t* col_idx, void* o, lcsa_strides os, float* lse, void* stream) {
  Geom g;
  lcsa_status st = validate_problem(p, &g);
  if (st != LCSA_OK) return st;
  const int64_t hw = int64_t(p->grid_h) * p->grid_w;
  if ((st = check_tensor("q", q, qs, p, hw * p->q_frames)) != LCSA_OK) return st;
  if ((st = check_tensor("k", k, ks, p, hw * p->kv_frames)) != LCSA_OK) return st;
  if ((st = check_tensor("v", v, vs, p, hw * p->kv_frames)) != LCSA_OK) return st;
  if ((st = check_tensor("o", o, os, p, hw * p->q_frames)) != LCSA_OK) return st;
  if (!row_ptr || !col_idx) return fail(LCSA_ERR_INVALID, "lcsa_attn_fwd: row_ptr or col_idx is NULL");
  if (reinterpret_cast<uintptr_t>(row_ptr) % 4 || reinterpret_cast<uintptr_t>(col_idx) % 4 ||
      reinterpret_cast<uintptr_t>(lse) % 4)
    return fail(LCSA_ERR_INVALID, "lcsa_attn_fwd: misaligned row_ptr, col_idx or lse");
  int32_t nnz = 0;
  if ((st = lcsa_csr_layout(p, nullptr, nullptr, &nnz, nullptr)) != LCSA_OK) return st;
  const int64_t esz = dtype_size(p);
  if ((hw * p->kv_frames * ks.token + p->head_dim) * esz >= (int64_t(1) << 32) ||
      (hw * p->kv_frames * vs.token + p->head_dim) * esz >= (int64_t(1) << 32))
    return fail(LCSA_ERR_UNSUPPORTED, "lcsa_attn_fwd: a per-head K or V span exceeds 4 GiB");
  AttnArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.row_ptr = row_ptr; a.col_idx = col_idx;
  a.qsb = qs.batch; a.qsh = qs.head; a.qst = qs.token;
  a.ksb = ks.batch; a.ksh = ks.head; a.kst = ks.token;
  a.vsb = vs.batch; a.vsh = vs.head; a.vst = vs.token;
  a.osb = os.batch; a.osh = os.head; a.ost = os.token;
  a.g = g;
  a.heads = p->heads;
  a.nnz = nnz;
  a.nq_tok = static_cast<int32_t>(hw * p->q_frames);
  a.nwg = p->batch * p->heads * g.nqb;
  a.c = static_cast<float>(static_cast<double>(p->scale) * 1.4426950408889634);
  a.k_span = static_cast<uint32_t>((hw * p->kv_frames - 1) * ks.token * esz + p->head_dim * esz);
  a.v_span = static_cast<uint32_t>((hw * p->kv_frames - 1) * vs.token * esz + p->head_dim * esz);
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (p->dtype == LCSA_BF16) {
    if (p->head_dim == 128) attn_fwd_direct_kernel<128><<<a.nwg, 256, 0, s>>>(a);
    else attn_fwd_direct_kernel<64><<<a.nwg, 256, 0, s>>>(a);
  } else {
    if (p->head_dim == 128) attn_fwd_kernel<float, 128><<<a.nwg, 256, 0, s>>>(a);
    else attn_fwd_kernel<float, 64><<<a.nwg, 256, 0, s>>>(a);
  }
  return hip_status(hipGetLastError(), "lcsa_attn_fwd launch");
}
