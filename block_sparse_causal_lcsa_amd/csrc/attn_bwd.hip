// lcsa_attn_bwd: gradients of the block-sparse attention (lcsa_attn_fwd) for a fixed selection.
// Stage 2 of FlashVSR trains the sparse-causal model with block-sparse attention (FlashVSR summary,
// sec. 2.2); training needs these gradients. For query token t of block i, the tokens k of its
// kept blocks, s = scale q.k, P = softmax(s) (recomputed from the forward's lse) and upstream dO:
//   dV_k += sum_t P_tk dO_t;  dP_tk = dO_t . v_k;  Delta_t = dO_t . O_t;  dS_tk = P_tk (dP_tk - Delta_t)
//   dQ_t = scale sum_k dS_tk k_k;  dK_k += scale sum_t dS_tk q_t.
// Kernels:
//   delta: Delta_t for every query token, and lse in log2 units (fp32, workspace).
//   csc:   per (batch, head), the transpose of the selection: for every key block the ascending list
//          of query blocks that kept it.
//   dq:    per (batch, head, query block), like the forward: 4 waves of 32 query rows (two
//          workgroups per CU), S^T = K Q^T and dP^T = V dO^T as bf16 MFMAs, dS^T in fp32,
//          dQ^T += K^T dS^T with dS^T rounded to bf16. K/V sub-tiles double-buffered in LDS.
//   dkdv:  per (batch, head, key block), over its query-block list: 4 waves of 32 key rows,
//          S = Q K^T and dP = dO V^T, then dV^T += dO^T P and dK^T += Q^T dS (P, dS rounded to bf16).
//          Q/dO sub-tiles and their lse/Delta in a 3-stage LDS pipeline.
// Every gradient element is written by exactly one workgroup, in a fixed order: results are
// deterministic and need no atomics. All operand tiles go from memory straight into LDS.
#include <hip/hip_runtime.h>

#include <math.h>

#include <mutex>
#include <utility>

#include "lcsa_internal.h"

namespace lcsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr int kTok = 64;                // tokens per tile: one latent frame of a 2x8x8 block
constexpr int kBufDword3 = 0x00020000;  // raw 32-bit buffer data format

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  int64_t qsb, qsh, qst, ksb, ksh, kst, vsb, vsh, vst, osb, osh, ost, dsb, dsh, dst;  // element strides
  const float* lse;        // [B*Hh, Nq] natural-log softmax denominators of the forward
  const int32_t* row_ptr;  // [nqb + 1]
  const int32_t* col_idx;  // [B*Hh, nnz], ascending per row
  float* dq;               // [B*Hh, Nq, d]
  float* dk;               // [B*Hh, Nk, d]
  float* dv;               // [B*Hh, Nk, d]
  float* delta;            // workspace [B*Hh, Nq]: rowsum(dO * O)
  float* lse2;             // workspace [B*Hh, Nq]: lse * log2(e)
  int32_t* col_ptr;        // workspace [B*Hh, nkb + 1]
  int32_t* row_of;         // workspace [B*Hh, nnz]
  Geom g;
  int32_t heads, nnz, nq_tok, nk_tok;
  float c;                 // scale * log2(e)
  float scale;
  uint32_t q_span, k_span, v_span, do_span;  // bytes of one (batch, head) slice
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), kBufDword3);
}

// Token index of row r (0..127) of block (tr, hb, wb), tr relative to the tensor's first temporal block.
__device__ __forceinline__ int block_token(const Geom& g, int tr, int hb, int wb, int r) {
  return ((kBlkT * tr + (r >> 6)) * g.H + kBlkH * hb + ((r >> 3) & 7)) * g.W + kBlkW * wb + (r & 7);
}

// Row r (0..127) of block (hb, wb): whether it lies inside the grid, and the row to read in its place
// when it does not (the nearest one inside, so every access stays in the tensor).
__device__ __forceinline__ bool row_inside(const Geom& g, int hb, int wb, int r, int* r_use) {
  const int rows = block_rows(g, hb), cols = block_cols(g, wb);
  const int y = (r >> 3) & 7, x = r & 7;
  *r_use = (r & 64) | ((y < rows ? y : rows - 1) << 3) | (x < cols ? x : cols - 1);
  return y < rows && x < cols;
}

// rows * 16 + cols inside the grid of block j (136 for a whole block).
__device__ __forceinline__ int block_lim(const Geom& g, int j) {
  const int rem = j % g.bpt;
  return 16 * block_rows(g, rem / g.Wb) + block_cols(g, rem % g.Wb);
}

// First token of block j (frame 0), for a tensor whose first temporal block is temporal block 0.
__device__ __forceinline__ uint32_t block_base(const Geom& g, int j) {
  const int tr = j / g.bpt, rem = j - (j / g.bpt) * g.bpt;
  const int hb = rem / g.Wb, wb = rem - (rem / g.Wb) * g.Wb;
  return uint32_t((kBlkT * tr * g.H + kBlkH * hb) * g.W + kBlkW * wb);
}

// A tile is 64 tokens x D bf16 in LDS, row-major; 16-byte chunk c of row r sits at chunk c ^ swz(r).
// Every tile is read two ways: row fragments (16 lanes on 16 consecutive rows, one chunk: needs swz
// to be a bijection on each aligned run of 16 rows) and ds_read_b64_tr_b16 fragments (4 aligned
// consecutive rows x 4 consecutive chunks per 32 lanes: needs the four swz values to differ in
// their upper two bits). For D = 128, swz(r) = 4 (r mod 4) + (r / 4) mod 4 does both; for D = 64
// (8 chunks per row) r mod 8 is used. Loads go straight to LDS.
template <int D>
__device__ __forceinline__ int swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : (r & 7);
}

template <int D>
struct TileB {
  static constexpr int CPR = D / 8;
  static constexpr int LOADS = kTok * CPR / 256;  // 16-byte loads per lane (256 lanes)
  static constexpr int ELEMS = kTok * D;
};

// Loads one tile with four waves; `wave` (0..3, wave-uniform) is this wave's share.
template <int D>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t rs, uint16_t* tile, uint32_t tst, uint32_t base_tok,
                                          int W, int wave) {
  constexpr int CPR = TileB<D>::CPR;
  // the scalar offset must be wave-uniform in registers the compiler can see as such
  const int lane = threadIdx.x & 63;
  wave = __builtin_amdgcn_readfirstlane(wave);
  base_tok = __builtin_amdgcn_readfirstlane(base_tok);
#pragma unroll
  for (int it = 0; it < TileB<D>::LOADS; ++it) {
    const int slot0 = (wave * TileB<D>::LOADS + it) * 64;
    const int r0 = slot0 / CPR;
    const int r = r0 + lane / CPR;
    const int c = (lane % CPR) ^ swz<D>(r);
    const uint32_t soff = (base_tok + uint32_t((r0 / 8) * W + (r0 % 8))) * tst * 2u;
    const uint32_t voff = (uint32_t(lane / CPR) * tst + 8u * uint32_t(c)) * 2u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (__attribute__((address_space(3))) void*)(tile + slot0 * 8), 16, voff, soff, 0, 0);
  }
}

// Row fragment: tile rows t*32 + l32, d = 16*s + 8*hi .. +8 (an MFMA A operand, or a B operand).
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const uint16_t* tile, int t, int s) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
  const int r = t * 32 + l32;
  return *reinterpret_cast<const bf16x8*>(tile + r * D + (((2 * s + hi) ^ swz<D>(r)) * 8));
}

// Transposed fragment: A operand [32 d x 16 tokens] of an MFMA whose k index runs over tile rows in
// the permuted order k-slot 8*hi + e <-> row t*32 + 16*h2 + 8*(e/4) + 4*hi + e%4 (the order in which
// a 32x32 score accumulator holds its rows), for d tile dt. Read with ds_read_b64_tr_b16.
template <int D>
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* tile, int t, int h2, int dt) {
  const int lane = threadIdx.x & 63, hi = lane >> 5, jj = lane & 15;
  const int vrow = 4 * hi + jj / 4, vcol = (lane & 16) + 4 * (jj & 3);
  v4i16 part[2];
#pragma unroll
  for (int e2 = 0; e2 < 2; ++e2) {
    const int row = t * 32 + 16 * h2 + 8 * e2 + vrow;
    const int col = dt * 32 + vcol;
    const uint16_t* p = tile + row * D + ((((col >> 3) ^ swz<D>(row)) << 3) | (col & 7));
    part[e2] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
  }
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Packs a 32x32 fp32 accumulator (rows in the MFMA result order) into two bf16 B operands whose
// k-slots follow the permuted order of tr_frag: half h2 holds items 8*h2 .. 8*h2 + 7.
__device__ __forceinline__ void pack_b(const f32x16& x, bf16x8 (&out)[2]) {
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int e = 0; e < 8; ++e) out[h2][e] = (__bf16)x[8 * h2 + e];
}

// Calls f(integral_constant<int, j>) for j = 0 .. N-1, fully unrolled with j a constant expression.
template <class F, int... J>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Wave-uniform 32-bit loads through the scalar cache (selection lists, row pointers).
typedef const __attribute__((address_space(4))) int32_t const_i32;

// Workgroup barrier without a memory fence: direct-to-LDS loads still in flight stay in flight
// (each wave waits for its own landed stages with vmcnt before). This wave's LDS reads are complete.
__device__ __forceinline__ void tile_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroup order: hardware deals workgroup n to XCD n % 8; each XCD gets a contiguous range so that
// neighbouring blocks of one head, which share most of their operands, share an L2.
__device__ __forceinline__ int xcd_order() {
  const int nwg = gridDim.x, n8 = (nwg / 8) * 8;
  const int wg = blockIdx.x;
  return wg < n8 ? (wg % 8) * (nwg / 8) + wg / 8 : wg;
}

// Waits until at most `ahead` stages of PER vector-memory ops each are still in flight (ahead <= 3).
template <int PER>
__device__ __forceinline__ void wait_stages(int ahead) {
  if (ahead >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * PER) : "memory");
  else if (ahead == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * PER) : "memory");
  else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(PER) : "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------------------- delta
template <int D>
__global__ __launch_bounds__(256) void delta_kernel(BwdArgs a, int64_t ntok) {
  constexpr int LPT = D / 8;             // lanes per token (8 elements each)
  constexpr int TPB = 256 / LPT;         // tokens per workgroup
  const int64_t t = int64_t(blockIdx.x) * TPB + threadIdx.x / LPT;
  const int c = threadIdx.x % LPT;
  float acc = 0.f;
  if (t < ntok) {
    const int64_t bh = t / a.nq_tok, n = t - bh * a.nq_tok;
    const int b = int(bh / a.heads), h = int(bh - (bh / a.heads) * a.heads);
    const uint4 ov = *reinterpret_cast<const uint4*>(a.o + b * a.osb + h * a.osh + n * a.ost + 8 * c);
    const uint4 gv = *reinterpret_cast<const uint4*>(a.dout + b * a.dsb + h * a.dsh + n * a.dst + 8 * c);
    const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc = __builtin_fmaf(__uint_as_float(ow[k] << 16), __uint_as_float(gw[k] << 16), acc);
      acc = __builtin_fmaf(__uint_as_float(ow[k] & 0xffff0000u), __uint_as_float(gw[k] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int o = LPT / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (t < ntok && c == 0) {
    a.delta[t] = acc;
    a.lse2[t] = a.lse[t] * 1.4426950408889634f;
  }
}

// ------------------------------------------------------------------------------------------ csc
// One workgroup per (batch, head). The kept (row, column) pairs of a range of columns are marked in
// an LDS bitmap stored column-major (column c owns words [c*wq, (c+1)*wq), bit i = query block i);
// each thread then counts and lists its own contiguous run of columns, so every list comes out in
// ascending row order whatever order the marks were set in.
constexpr int kCscWords = 16384;  // 64 KB bitmap

__global__ __launch_bounds__(1024) void csc_kernel(BwdArgs a) {
  __shared__ uint32_t bits[kCscWords];
  __shared__ int32_t part[1024];
  const Geom& g = a.g;
  const int bh = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int32_t* col = a.col_idx + int64_t(bh) * a.nnz;
  int32_t* cp = a.col_ptr + int64_t(bh) * (g.nkb + 1);
  int32_t* ro = a.row_of + int64_t(bh) * a.nnz;
  const int wq = (g.nqb + 31) / 32;  // bitmap words per column (the host checks wq <= kCscWords)
  const int cw = kCscWords / wq;     // columns per pass
  if (threadIdx.x == 0) cp[0] = 0;
  int base = 0;                      // entries listed by earlier passes
  for (int c0 = 0; c0 < g.nkb; c0 += cw) {
    const int nc = min(cw, g.nkb - c0);
    for (int w = threadIdx.x; w < nc * wq; w += 1024) bits[w] = 0;
    __syncthreads();
    // one wave per query block, lanes over its kept entries
    for (int i = wave; i < g.nqb; i += 16) {
      const int rb = a.row_ptr[i], re = a.row_ptr[i + 1];
      for (int e = rb + lane; e < re; e += 64) {
        const int c = col[e] - c0;
        if (c >= 0 && c < nc) atomicOr(&bits[c * wq + (i >> 5)], 1u << (i & 31));
      }
    }
    __syncthreads();
    const int per = (nc + 1023) / 1024;
    const int cb = min(int(threadIdx.x) * per, nc), ce = min(cb + per, nc);
    int cnt = 0;
    for (int c = cb; c < ce; ++c)
      for (int w = 0; w < wq; ++w) cnt += __popc(bits[c * wq + w]);
    // inclusive scan of the per-thread counts (Hillis-Steele over 1024 entries)
    part[threadIdx.x] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int x = int(threadIdx.x) >= off ? part[threadIdx.x - off] : 0;
      __syncthreads();
      part[threadIdx.x] += x;
      __syncthreads();
    }
    int run = base + part[threadIdx.x] - cnt;
    const int pass_total = part[1023];
    for (int c = cb; c < ce; ++c) {
      for (int w = 0; w < wq; ++w) {
        uint32_t m = bits[c * wq + w];
        while (m) {
          ro[run++] = 32 * w + __builtin_ctz(m);
          m &= m - 1;
        }
      }
      cp[c0 + c + 1] = run;
    }
    base += pass_total;
    __syncthreads();  // the next pass clears the bitmap and reuses part
  }
}

// ------------------------------------------------------------------------------------------- dq
// MASK: kMaskNone (whole blocks, block-granular windows: no token mask); kMaskRagged (the grid is
// not a multiple of 8: partial edge blocks mask their missing keys and query rows); kMaskWindow
// (token-granular window: per-token masks in blocks not seen whole by every query token; rows that
// see no key have lse = -inf and get P = 0).
constexpr int kMaskNone = 0, kMaskRagged = 1, kMaskWindow = 2;

template <int D, int MASK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void dq_kernel(BwdArgs a) {
  constexpr int DS = D / 16, DT = D / 32;
  constexpr int TE = TileB<D>::ELEMS;
  __shared__ __attribute__((aligned(16))) uint16_t kbuf[2 * TE];
  __shared__ __attribute__((aligned(16))) uint16_t vbuf[2 * TE];
  const Geom& g = a.g;
  const int bh = xcd_order() / g.nqb, i = xcd_order() - bh * g.nqb;
  const int b = bh / a.heads, h = bh - (bh / a.heads) * a.heads;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l32 = lane & 31, hi = lane >> 5;
  const int qtr = i / g.bpt, qrem = i - (i / g.bpt) * g.bpt;
  const int qhb = qrem / g.Wb, qwb = qrem - (qrem / g.Wb) * g.Wb;
  int qrow = 32 * wave + l32;
  const bool q_in = MASK != kMaskNone ? row_inside(g, qhb, qwb, 32 * wave + l32, &qrow) : true;
  const int qtok = block_token(g, qtr, qhb, qwb, qrow);
  int lo_h = 0, hi_h = 0, lo_w = 0, hi_w = 0;  // this lane's query token window (kMaskWindow)
  if constexpr (MASK == kMaskWindow) {
    const bool pres = g.win_mode == kWinTokenPreserving;
    tok_range(pres, kBlkH * qhb + ((qrow >> 3) & 7), g.H, g.wth, &lo_h, &hi_h);
    tok_range(pres, kBlkW * qwb + (qrow & 7), g.W, g.wtw, &lo_w, &hi_w);
  }

  bf16x8 qf[DS], gf[DS];  // B operands: this lane's query row, d = 16*s + 8*hi .. +8
  {
    const uint16_t* qs = a.q + b * a.qsb + h * a.qsh + int64_t(qtok) * a.qst + 8 * hi;
    const uint16_t* gs = a.dout + b * a.dsb + h * a.dsh + int64_t(qtok) * a.dst + 8 * hi;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      qf[s] = *reinterpret_cast<const bf16x8*>(qs + 16 * s);
      gf[s] = *reinterpret_cast<const bf16x8*>(gs + 16 * s);
    }
  }
  const float lse2 = a.lse2[int64_t(bh) * a.nq_tok + qtok];
  const float dlt = a.delta[int64_t(bh) * a.nq_tok + qtok];
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k + b * a.ksb + h * a.ksh, a.k_span);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.v + b * a.vsb + h * a.vsh, a.v_span);
  const uint32_t kst = uint32_t(a.kst), vst = uint32_t(a.vst);
  const uint32_t hw = uint32_t(g.H) * uint32_t(g.W);
  const const_i32* rp = (const const_i32*)(a.row_ptr);
  const int beg = rp[i], nsel = rp[i + 1] - beg;
  const const_i32* sel = (const const_i32*)(a.col_idx) + int64_t(bh) * a.nnz + beg;

  f32x16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  // sub-tile m = frame m%2 of entry m/2; invalid entries load block 0 and contribute nothing
  auto base_of = [&](int m, bool& ok, int& lim) -> uint32_t {
    const int j = sel[m >> 1];
    ok = j >= 0 && j < g.nkb;
    if constexpr (MASK == kMaskRagged) lim = block_lim(g, ok ? j : 0);
    if constexpr (MASK == kMaskWindow) {
      const int jj = ok ? j : 0, rem = jj % g.bpt, hb = rem / g.Wb, wb = rem % g.Wb;
      lim = block_seen_whole(g, qhb, qwb, hb, wb) ? -1 : ((hb << 16) | wb);
    }
    return block_base(g, ok ? j : 0) + uint32_t(m & 1) * hw;
  };
  // One 64-key sub-tile = two 32-key tiles t, one at a time: S^T = K Q^T and dP^T = V dO^T, the vector
  // step dS^T = P^T (dP^T - Delta), then dQ^T += K^T dS^T. At two waves per SIMD the other wave fills
  // the gaps; an explicit MFMA list with operands read ahead (as in the dK/dV kernel) needs more
  // registers than two waves leave and was slower.
  auto step = [&](const uint16_t* Kt, const uint16_t* Vt, bool ok, int lim) __attribute__((always_inline)) {
    // a skipped entry, or a row that sees no key (lse = -inf), gives P = dS = 0
    const float neg = ok && lse2 != -INFINITY ? -lse2 : -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x16 st = f32x16{}, pt = f32x16{};
#pragma unroll
      for (int s = 0; s < DS; ++s) {
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(Kt, t, s), qf[s], st, 0, 0, 0);
        pt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(Vt, t, s), gf[s], pt, 0, 0, 0);
      }
      if constexpr (MASK == kMaskRagged) {
        if (lim != 16 * kBlkH + kBlkW) mask_partial_tile(st, t, hi, lim >> 4, lim & 15);  // keys outside the grid
      }
      if constexpr (MASK == kMaskWindow) {
        if (lim >= 0)  // keys outside this query token's window
          mask_window_tile(st, t, hi, kBlkH * (lim >> 16), kBlkW * (lim & 0xffff), lo_h, hi_h, lo_w, hi_w);
      }
      f32x16 d;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(st[v], a.c, neg));
        d[v] = p * (pt[v] - dlt);
      }
      bf16x8 dsf[2];
      pack_b(d, dsf);
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_frag<D>(Kt, t, h2, dt), dsf[h2], acc[dt], 0, 0, 0);
    }
  };

  // sub-tile m lives in buffer m % 2; the loads of m + 1 run while m is computed (two workgroups
  // per CU hide the rest of the load latency)
  const int total = 2 * nsel;
  bool ok_c = false, ok_n = false;
  int lim_c = 136, lim_n = 136;
  if (total > 0) {
    const uint32_t b0 = base_of(0, ok_n, lim_n);
    load_tile<D>(krs, kbuf, kst, b0, g.W, wave);
    load_tile<D>(vrs, vbuf, vst, b0, g.W, wave);
  }
  for (int m = 0; m < total; ++m) {
    ok_c = ok_n;
    lim_c = lim_n;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    tile_barrier();
    if (m + 1 < total) {
      const uint32_t bn = base_of(m + 1, ok_n, lim_n);
      load_tile<D>(krs, kbuf + ((m + 1) & 1) * TE, kst, bn, g.W, wave);
      load_tile<D>(vrs, vbuf + ((m + 1) & 1) * TE, vst, bn, g.W, wave);
    }
    step(kbuf + (m & 1) * TE, vbuf + (m & 1) * TE, ok_c, lim_c);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (!q_in) return;  // a query row outside the grid (partial block) has no gradient

  float* out = a.dq + (int64_t(bh) * a.nq_tok + qtok) * D;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = dt * 32 + 8 * g4 + 4 * hi;
      *reinterpret_cast<float4*>(out + d0) =
          make_float4(acc[dt][4 * g4] * a.scale, acc[dt][4 * g4 + 1] * a.scale, acc[dt][4 * g4 + 2] * a.scale,
                      acc[dt][4 * g4 + 3] * a.scale);
    }
}

// ----------------------------------------------------------------------------------------- dkdv
// dK/dV with two waves per key tile on one SIMD (8 waves, 512 lanes, 128 keys per workgroup): role 0
// (waves 0-3) computes S = Q K^T, P = 2^(c S - lse2) and dV^T += dO^T P; role 1 (waves 4-7) computes
// dP = dO V^T, dS = P (dP - Delta) and dK^T += Q^T dS, with P passed from its partner through LDS.
// Each wave holds one accumulator set (dV or dK) and one operand set (K or V), so two waves fit a
// SIMD and one wave's vector work overlaps the other's matrix work. Two barriers per sub-tile:
// the first publishes the sub-tile's Q/dO tiles, the second the probabilities.
template <int D, int MASK>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void dkdv_split_kernel(BwdArgs a) {
  constexpr int DS = D / 16, DT = D / 32;
  constexpr int TE = TileB<D>::ELEMS;
  constexpr int kLook = 4;
  __shared__ __attribute__((aligned(16))) uint16_t qbuf[2 * TE];
  __shared__ __attribute__((aligned(16))) uint16_t gbuf[2 * TE];
  __shared__ __attribute__((aligned(16))) float rlbuf[2 * 2 * kTok];   // per stage: [lse2 | delta]
  // per key tile: P as [lane][kPRow] floats, items (t, v) at t * 16 + v; the padded row makes the
  // 16-byte accesses of 16 consecutive lanes cover all 64 banks once
  constexpr int kPRow = 36;
  __shared__ __attribute__((aligned(16))) float pbuf[4 * 64 * kPRow];
  const Geom& g = a.g;
  const int bh = xcd_order() / g.nkb, j = xcd_order() - bh * g.nkb;
  const int b = bh / a.heads, h = bh - (bh / a.heads) * a.heads;
  const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int role = wave >> 2, kr = wave & 3;       // role 0: S, P, dV; role 1: dP, dS, dK; key tile kr
  const int ktr = j / g.bpt, krem = j - (j / g.bpt) * g.bpt;
  const int khb = krem / g.Wb, kwb = krem - (krem / g.Wb) * g.Wb;
  int krow = 32 * kr + l32;
  const bool k_in = MASK != kMaskNone ? row_inside(g, khb, kwb, 32 * kr + l32, &krow) : true;
  const int ktok = block_token(g, ktr, khb, kwb, krow);
  const int hk = kBlkH * khb + ((krow >> 3) & 7), wk = kBlkW * kwb + (krow & 7);  // this lane's key token

  bf16x8 opf[DS];  // B operands: this lane's key row of K (role 0) or V (role 1)
  {
    const uint16_t* src = role == 0 ? a.k + b * a.ksb + h * a.ksh + int64_t(ktok) * a.kst
                                    : a.v + b * a.vsb + h * a.vsh + int64_t(ktok) * a.vst;
#pragma unroll
    for (int s = 0; s < DS; ++s) opf[s] = *reinterpret_cast<const bf16x8*>(src + 8 * hi + 16 * s);
  }
  // role 0 loads the Q tiles and lse2, role 1 the dO tiles and Delta
  const __amdgpu_buffer_rsrc_t trs = role == 0 ? make_rsrc(a.q + b * a.qsb + h * a.qsh, a.q_span)
                                               : make_rsrc(a.dout + b * a.dsb + h * a.dsh, a.do_span);
  const uint32_t tst = role == 0 ? uint32_t(a.qst) : uint32_t(a.dst);
  const float* rsrc = role == 0 ? a.lse2 : a.delta;
  const __amdgpu_buffer_rsrc_t rrs = make_rsrc(rsrc + int64_t(bh) * a.nq_tok, uint32_t(a.nq_tok) * 4u);
  uint16_t* tbuf = role == 0 ? qbuf : gbuf;
  const uint32_t hw = uint32_t(g.H) * uint32_t(g.W);
  const const_i32* cp = (const const_i32*)(a.col_ptr) + int64_t(bh) * (g.nkb + 1);
  const int beg = cp[j], nrow = cp[j + 1] - beg;
  const const_i32* rows = (const const_i32*)(a.row_of) + int64_t(bh) * a.nnz + beg;
  float* pmine = pbuf + kr * (64 * kPRow) + lane * kPRow;

  f32x16 acc[DT];  // dV^T (role 0) or dK^T (role 1)
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x16{};

  auto qbase_of = [&](int m) -> uint32_t {
    const int i = rows[m >> 1];
    const int tr = i / g.bpt, rem = i - (i / g.bpt) * g.bpt;
    const int hb = rem / g.Wb, wb = rem - (rem / g.Wb) * g.Wb;
    return uint32_t((kBlkT * tr * g.H + kBlkH * hb) * g.W + kBlkW * wb) + uint32_t(m & 1) * hw;
  };
  auto issue = [&](int m) {
    const int sb = m & 1;
    const uint32_t bn = __builtin_amdgcn_readfirstlane(qbase_of(m));
    load_tile<D>(trs, tbuf + sb * TE, tst, bn, g.W, kr);
    float* rl = rlbuf + sb * 2 * kTok + role * kTok + 16 * kr;
    if (lane < 16) {
      const int r = 16 * kr + lane;
      const uint32_t voff = uint32_t((r >> 3) * g.W + (r & 7)) * 4u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rrs, (__attribute__((address_space(3))) void*)(rl), 4, voff,
                                               bn * 4u, 0, 0);
    }
  };
  // item v of tile t of a score accumulator is query row t*32 + (v/4)*8 + 4*hi + v%4 of the sub-tile
  auto mask_rows = [&](f32x16& x, int t, int lim) __attribute__((always_inline)) {
    if constexpr (MASK == kMaskRagged) {
      if (lim != 16 * kBlkH + kBlkW) mask_partial_tile(x, t, hi, lim >> 4, lim & 15);
    }
    if constexpr (MASK == kMaskWindow) {
      if (lim >= 0) mask_window_tile_q(x, t, hi, kBlkH * (lim >> 16), kBlkW * (lim & 0xffff), hk, wk, g);
    }
  };
  // NA = 2 * DS products of the first phase (tile t = o / DS, d step o % DS) and NB = 4 * DT of the
  // second (tile t = o / (2 DT), half h2 = (o / DT) & 1, d tile o % DT), operands read kLook ahead
  constexpr int NA = 2 * DS, NB = 4 * DT;
  auto phase1 = [&](const uint16_t* T, f32x16 (&x)[2]) __attribute__((always_inline)) {
    x[0] = x[1] = f32x16{};
    bf16x8 fr[kLook];
    static_for<kLook>([&](auto jc) __attribute__((always_inline)) {
      constexpr int o = decltype(jc)::value;
      fr[o] = row_frag<D>(T, o / DS, o % DS);
    });
    static_for<NA>([&](auto jc) __attribute__((always_inline)) {
      constexpr int o = decltype(jc)::value;
      const bf16x8 f = fr[o % kLook];
      if constexpr (o + kLook < NA) fr[o % kLook] = row_frag<D>(T, (o + kLook) / DS, (o + kLook) % DS);
      x[o / DS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, opf[o % DS], x[o / DS], 0, 0, 0);
    });
  };
  auto phase2 = [&](const uint16_t* T, const bf16x8 (&bop)[2][2]) __attribute__((always_inline)) {
    bf16x8 fr[kLook];
    static_for<kLook>([&](auto jc) __attribute__((always_inline)) {
      constexpr int o = decltype(jc)::value;
      fr[o] = tr_frag<D>(T, o / (2 * DT), (o / DT) & 1, o % DT);
    });
    static_for<NB>([&](auto jc) __attribute__((always_inline)) {
      constexpr int o = decltype(jc)::value;
      const bf16x8 f = fr[o % kLook];
      if constexpr (o + kLook < NB)
        fr[o % kLook] = tr_frag<D>(T, (o + kLook) / (2 * DT), ((o + kLook) / DT) & 1, (o + kLook) % DT);
      acc[o % DT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f, bop[o / (2 * DT)][(o / DT) & 1], acc[o % DT], 0, 0, 0);
    });
  };

  const int total = 2 * nrow;
  if (total > 0) issue(0);
  for (int m = 0; m < total; ++m) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // stage m has landed for this wave
    tile_barrier();                                    // ... for every wave; stage m - 1 and P are free
    if (m + 1 < total) issue(m + 1);
    const int sb = m & 1;
    const uint16_t* Qt = qbuf + sb * TE;
    const uint16_t* Gt = gbuf + sb * TE;
    const float* rl = rlbuf + sb * 2 * kTok;
    int lim = 136;
    if constexpr (MASK == kMaskRagged) lim = block_lim(g, rows[m >> 1]);
    if constexpr (MASK == kMaskWindow) {
      const int qi = rows[m >> 1], rem = qi % g.bpt, qhb = rem / g.Wb, qwb = rem % g.Wb;
      lim = block_seen_whole(g, qhb, qwb, khb, kwb) && block_rows(g, qhb) == kBlkH && block_cols(g, qwb) == kBlkW
                ? -1 : ((qhb << 16) | qwb);
    }
    f32x16 x[2];
    bf16x8 bop[2][2];
    if (role == 0) {
      phase1(Qt, x);  // S = Q K^T
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        mask_rows(x[t], t, lim);
        f32x16 pv;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 l4 = *reinterpret_cast<const float4*>(rl + t * 32 + g4 * 8 + 4 * hi);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // a query row that sees no key (lse = -inf) gets P = 0
            const float nl = MASK == kMaskWindow && lv[e] == -INFINITY ? -INFINITY : -lv[e];
            pv[4 * g4 + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[t][4 * g4 + e], a.c, nl));
          }
        }
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
          *reinterpret_cast<float4*>(pmine + t * 16 + 4 * v4) =
              make_float4(pv[4 * v4], pv[4 * v4 + 1], pv[4 * v4 + 2], pv[4 * v4 + 3]);
        pack_b(pv, bop[t]);
      }
      tile_barrier();    // P published
      phase2(Gt, bop);   // dV^T += dO^T P
    } else {
      phase1(Gt, x);     // dP = dO V^T
      tile_barrier();    // P published
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        f32x16 ds;
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 d4 = *reinterpret_cast<const float4*>(rl + kTok + t * 32 + g4 * 8 + 4 * hi);
          const float4 p4 = *reinterpret_cast<const float4*>(pmine + t * 16 + 4 * g4);
          const float dv4[4] = {d4.x, d4.y, d4.z, d4.w}, pv4[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * g4 + e;
            ds[v] = pv4[e] * (x[t][v] - dv4[e]);
          }
        }
        pack_b(ds, bop[t]);
      }
      phase2(Qt, bop);   // dK^T += Q^T dS
    }
  }

  if (!k_in) return;  // a key row outside the grid (partial block) has no gradient
  float* out = (role == 0 ? a.dv : a.dk) + (int64_t(bh) * a.nk_tok + ktok) * D;
  const float sc = role == 0 ? 1.f : a.scale;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = dt * 32 + 8 * g4 + 4 * hi;
      *reinterpret_cast<float4*>(out + d0) =
          make_float4(acc[dt][4 * g4] * sc, acc[dt][4 * g4 + 1] * sc, acc[dt][4 * g4 + 2] * sc, acc[dt][4 * g4 + 3] * sc);
    }
}

struct BwdLayout {
  size_t delta, lse2, col_ptr, row_of, total;
};

BwdLayout bwd_layout(const lcsa_problem* p, const Geom& g, int32_t nnz) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t bhn = size_t(p->batch) * p->heads;
  BwdLayout l{};
  l.delta = 0;
  l.lse2 = up(bhn * size_t(g.nqb) * kBlkTokens * sizeof(float));
  l.col_ptr = l.lse2 + up(bhn * size_t(g.nqb) * kBlkTokens * sizeof(float));
  l.row_of = l.col_ptr + up(bhn * size_t(g.nkb + 1) * sizeof(int32_t));
  l.total = l.row_of + up(bhn * size_t(nnz > 0 ? nnz : 1) * sizeof(int32_t));
  return l;
}

// Workspace of lcsa_attn_bwd_noalloc: one static device array per GPU, held until the process ends.
// Host code never passes `scratch` itself to a kernel (in host code the name is a host-side shadow,
// not a device address); it uses the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[LCSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device.
lcsa_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "lcsa_attn_bwd_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(LCSA_ERR_UNSUPPORTED, "lcsa_attn_bwd_noalloc: device %d beyond the %d supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "lcsa_attn_bwd_noalloc: hipGetSymbolAddress(scratch)");
    if (!ptr || reinterpret_cast<uintptr_t>(ptr) % 256)
      return fail(LCSA_ERR_HIP, "lcsa_attn_bwd_noalloc: scratch address %p is not 256-byte aligned", ptr);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LCSA_OK;
}

// Both backward entry points: validation, then the four launches. With use_scratch the workspace
// is this device's static scratch array (workspace and workspace_bytes are ignored).
lcsa_status attn_bwd_run(const lcsa_problem* p, const void* q, lcsa_strides qs, const void* k, lcsa_strides ks,
                         const void* v, lcsa_strides vs, const void* o, lcsa_strides os, const void* d_o,
                         lcsa_strides dos, const float* lse, const int32_t* row_ptr, const int32_t* col_idx,
                         float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream,
                         bool use_scratch);

}  // namespace
}  // namespace lcsa

using namespace lcsa;

extern "C" lcsa_status lcsa_attn_bwd_workspace_size(const lcsa_problem* p, size_t* bytes) {
  Geom g;
  lcsa_status st = validate_problem(p, &g);
  if (st != LCSA_OK) return st;
  if (!bytes) return fail(LCSA_ERR_INVALID, "lcsa_attn_bwd_workspace_size: bytes is NULL");
  int32_t nnz = 0;
  if ((st = lcsa_csr_layout(p, nullptr, nullptr, &nnz, nullptr)) != LCSA_OK) return st;
  *bytes = bwd_layout(p, g, nnz).total;
  return LCSA_OK;
}

extern "C" lcsa_status lcsa_attn_bwd(const lcsa_problem* p, const void* q, lcsa_strides qs, const void* k,
                                     lcsa_strides ks, const void* v, lcsa_strides vs, const void* o, lcsa_strides os,
                                     const void* d_o, lcsa_strides dos, const float* lse, const int32_t* row_ptr,
                                     const int32_t* col_idx, float* dq, float* dk, float* dv, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return attn_bwd_run(p, q, qs, k, ks, v, vs, o, os, d_o, dos, lse, row_ptr, col_idx, dq, dk, dv, workspace,
                      workspace_bytes, stream, false);
}

extern "C" lcsa_status lcsa_attn_bwd_noalloc(const lcsa_problem* p, const void* q, lcsa_strides qs, const void* k,
                                             lcsa_strides ks, const void* v, lcsa_strides vs, const void* o,
                                             lcsa_strides os, const void* d_o, lcsa_strides dos, const float* lse,
                                             const int32_t* row_ptr, const int32_t* col_idx, float* dq, float* dk,
                                             float* dv, void* stream) {
  return attn_bwd_run(p, q, qs, k, ks, v, vs, o, os, d_o, dos, lse, row_ptr, col_idx, dq, dk, dv, nullptr, 0,
                      stream, true);
}

namespace lcsa {
namespace {

lcsa_status attn_bwd_run(const lcsa_problem* p, const void* q, lcsa_strides qs, const void* k, lcsa_strides ks,
                         const void* v, lcsa_strides vs, const void* o, lcsa_strides os, const void* d_o,
                         lcsa_strides dos, const float* lse, const int32_t* row_ptr, const int32_t* col_idx,
                         float* dq, float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream,
                         bool use_scratch) {
  Geom g;
  lcsa_status st = validate_problem(p, &g);
  if (st != LCSA_OK) return st;
  if (p->dtype != LCSA_BF16) return fail(LCSA_ERR_UNSUPPORTED, "lcsa_attn_bwd: only bf16 inputs are implemented");
  const int64_t hw = int64_t(p->grid_h) * p->grid_w;
  if ((st = check_tensor("q", q, qs, p, hw * p->q_frames)) != LCSA_OK) return st;
  if ((st = check_tensor("k", k, ks, p, hw * p->kv_frames)) != LCSA_OK) return st;
  if ((st = check_tensor("v", v, vs, p, hw * p->kv_frames)) != LCSA_OK) return st;
  if ((st = check_tensor("o", o, os, p, hw * p->q_frames)) != LCSA_OK) return st;
  if ((st = check_tensor("d_o", d_o, dos, p, hw * p->q_frames)) != LCSA_OK) return st;
  if (!lse || !row_ptr || !col_idx || !dq || !dk || !dv || (!workspace && !use_scratch))
    return fail(LCSA_ERR_INVALID, "lcsa_attn_bwd: NULL lse, row_ptr, col_idx, gradient or workspace");
  if (reinterpret_cast<uintptr_t>(lse) % 4 || reinterpret_cast<uintptr_t>(row_ptr) % 4 ||
      reinterpret_cast<uintptr_t>(col_idx) % 4 || reinterpret_cast<uintptr_t>(dq) % 16 ||
      reinterpret_cast<uintptr_t>(dk) % 16 || reinterpret_cast<uintptr_t>(dv) % 16 ||
      (!use_scratch && reinterpret_cast<uintptr_t>(workspace) % 256))
    return fail(LCSA_ERR_INVALID, "lcsa_attn_bwd: misaligned lse, row_ptr, col_idx, gradient or workspace");
  if ((g.nqb + 31) / 32 > kCscWords)
    return fail(LCSA_ERR_UNSUPPORTED, "lcsa_attn_bwd: more than %d query blocks per head", 32 * kCscWords);
  int32_t nnz = 0;
  if ((st = lcsa_csr_layout(p, nullptr, nullptr, &nnz, nullptr)) != LCSA_OK) return st;
  const BwdLayout l = bwd_layout(p, g, nnz);
  if (use_scratch) {
    if (l.total > size_t(LCSA_NOALLOC_SCRATCH_BYTES))
      return fail(LCSA_ERR_UNSUPPORTED,
                  "lcsa_attn_bwd_noalloc: the problem needs %zu bytes of workspace, more than the %zu-byte "
                  "static scratch buffer (use lcsa_attn_bwd with a caller workspace)",
                  l.total, size_t(LCSA_NOALLOC_SCRATCH_BYTES));
  } else if (workspace_bytes < l.total) {
    return fail(LCSA_ERR_INVALID, "lcsa_attn_bwd: workspace of %zu bytes, %zu needed", workspace_bytes, l.total);
  }
  const int64_t esz = 2;
  auto span = [&](lcsa_strides s, int64_t ntok) { return (ntok - 1) * s.token * esz + p->head_dim * esz; };
  if (span(qs, hw * p->q_frames) >= (int64_t(1) << 32) || span(ks, hw * p->kv_frames) >= (int64_t(1) << 32) ||
      span(vs, hw * p->kv_frames) >= (int64_t(1) << 32) || span(dos, hw * p->q_frames) >= (int64_t(1) << 32))
    return fail(LCSA_ERR_UNSUPPORTED, "lcsa_attn_bwd: a per-head tensor span exceeds 4 GiB");

  BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(d_o);
  a.qsb = qs.batch; a.qsh = qs.head; a.qst = qs.token;
  a.ksb = ks.batch; a.ksh = ks.head; a.kst = ks.token;
  a.vsb = vs.batch; a.vsh = vs.head; a.vst = vs.token;
  a.osb = os.batch; a.osh = os.head; a.ost = os.token;
  a.dsb = dos.batch; a.dsh = dos.head; a.dst = dos.token;
  a.lse = lse;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.g = g;
  a.heads = p->heads;
  a.nnz = nnz;
  a.nq_tok = static_cast<int32_t>(hw * p->q_frames);
  a.nk_tok = static_cast<int32_t>(hw * p->kv_frames);
  a.scale = p->scale;
  a.c = static_cast<float>(static_cast<double>(p->scale) * 1.4426950408889634);
  a.q_span = static_cast<uint32_t>(span(qs, hw * p->q_frames));
  a.k_span = static_cast<uint32_t>(span(ks, hw * p->kv_frames));
  a.v_span = static_cast<uint32_t>(span(vs, hw * p->kv_frames));
  a.do_span = static_cast<uint32_t>(span(dos, hw * p->q_frames));
  if (use_scratch) {  // every check has passed: only now touch HIP for the scratch address
    if ((st = scratch_for_current_device(&workspace)) != LCSA_OK) return st;
  }
  char* w = static_cast<char*>(workspace);
  a.delta = reinterpret_cast<float*>(w + l.delta);
  a.lse2 = reinterpret_cast<float*>(w + l.lse2);
  a.col_ptr = reinterpret_cast<int32_t*>(w + l.col_ptr);
  a.row_of = reinterpret_cast<int32_t*>(w + l.row_of);

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int bhn = p->batch * p->heads;
  const int64_t ntok = int64_t(bhn) * a.nq_tok;
  if (p->head_dim == 128) {
    delta_kernel<128><<<int((ntok + 15) / 16), 256, 0, s>>>(a, ntok);
  } else {
    delta_kernel<64><<<int((ntok + 31) / 32), 256, 0, s>>>(a, ntok);
  }
  csc_kernel<<<bhn, 1024, 0, s>>>(a);
  const bool ragged = (g.H % kBlkH) != 0 || (g.W % kBlkW) != 0;
  const int mask = token_window(g) ? kMaskWindow : (ragged ? kMaskRagged : kMaskNone);
#define DKDV_LAUNCH(DD, MM) dkdv_split_kernel<DD, MM><<<bhn * g.nkb, 512, 0, s>>>(a)
  if (p->head_dim == 128) {
    if (mask == kMaskWindow) {
      dq_kernel<128, kMaskWindow><<<bhn * g.nqb, 256, 0, s>>>(a);
      DKDV_LAUNCH(128, kMaskWindow);
    } else if (mask == kMaskRagged) {
      dq_kernel<128, kMaskRagged><<<bhn * g.nqb, 256, 0, s>>>(a);
      DKDV_LAUNCH(128, kMaskRagged);
    } else {
      dq_kernel<128, kMaskNone><<<bhn * g.nqb, 256, 0, s>>>(a);
      DKDV_LAUNCH(128, kMaskNone);
    }
  } else {
    if (mask == kMaskWindow) {
      dq_kernel<64, kMaskWindow><<<bhn * g.nqb, 256, 0, s>>>(a);
      DKDV_LAUNCH(64, kMaskWindow);
    } else if (mask == kMaskRagged) {
      dq_kernel<64, kMaskRagged><<<bhn * g.nqb, 256, 0, s>>>(a);
      DKDV_LAUNCH(64, kMaskRagged);
    } else {
      dq_kernel<64, kMaskNone><<<bhn * g.nqb, 256, 0, s>>>(a);
      DKDV_LAUNCH(64, kMaskNone);
    }
  }
  return hip_status(hipGetLastError(), "lcsa_attn_bwd launch");
}

}  // namespace
}  // namespace lcsa
