// lcsa_pool: mean of every 2x8x8 token block of Q and K (FlashVSR summary, sec. 2.2: Q and K are
// average-pooled per block into compact block features). Edge blocks of a grid that is not a
// multiple of 8 are partial and averaged over the tokens they have.
//
// One workgroup (256 lanes) per (batch, head, block). A block is 16 rows of 8 consecutive tokens;
// each lane owns one 16-byte chunk of a token row and walks the block's tokens with a fixed stride,
// so a wave reads whole contiguous token rows (64 x 16 B). Sums are kept in fp64, which makes the
// block sum of bf16 inputs exact; the mean is rounded once to fp32. Pure streaming: every input
// byte is read once, 4*d bytes are written per block.
#include <hip/hip_runtime.h>

#include "lcsa_internal.h"

namespace lcsa {
namespace {

struct PoolTensor {
  const void* x;
  int64_t sb, sh, st;  // element strides: batch, head, token
  float* out;          // block b of (batch, head) bh at row bh * out_rows + out_off + b, d floats each
  int32_t nblk;
  int32_t wgs;         // workgroups assigned to this tensor = B * Hh * nblk
  int32_t out_rows, out_off;
};

// RAGGED: the grid is not a multiple of 8 and edge blocks are partial.
template <typename T, int D, bool RAGGED>
__global__ __launch_bounds__(256) void pool_kernel(PoolTensor ta, PoolTensor tb, int heads, Geom g) {
  constexpr int EPC = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte chunk
  constexpr int CPT = D / EPC;                           // chunks per token row
  constexpr int SLOTS = 256 / CPT;                       // lanes sharing a chunk column
  constexpr int TPS = kBlkTokens / SLOTS;                // tokens per lane
  __shared__ double part[SLOTS][D];

  int wg = blockIdx.x;
  const bool second = wg >= ta.wgs;
  const PoolTensor t = second ? tb : ta;
  if (second) wg -= ta.wgs;

  const int blk = wg % t.nblk;
  const int bh = wg / t.nblk;
  const int b = bh / heads, h = bh - (bh / heads) * heads;
  const int tr = blk / g.bpt, rem = blk - (blk / g.bpt) * g.bpt;
  const int hb = rem / g.Wb, wb = rem - (rem / g.Wb) * g.Wb;
  const T* base = static_cast<const T*>(t.x) + b * t.sb + h * t.sh;
  // a block in the last block row / column of a grid that is not a multiple of 8 is partial
  const int rows = RAGGED ? block_rows(g, hb) : kBlkH, cols = RAGGED ? block_cols(g, wb) : kBlkW;

  const int c = threadIdx.x % CPT;
  const int slot = threadIdx.x / CPT;

  uint4 raw[TPS];
#pragma unroll
  for (int k = 0; k < TPS; ++k) {
    const int tok = slot + k * SLOTS;  // 0..127: (frame, row, col) = (tok/64, tok/8%8, tok%8)
    const int64_t n = (int64_t(kBlkT * tr + tok / 64) * g.H + kBlkH * hb + (tok / 8) % 8) * g.W +
                      kBlkW * wb + tok % 8;
    const bool in = !RAGGED || ((tok / 8) % 8 < rows && tok % 8 < cols);
    raw[k] = in ? *reinterpret_cast<const uint4*>(base + n * t.st + c * EPC) : make_uint4(0, 0, 0, 0);
  }
  double acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0;
#pragma unroll
  for (int k = 0; k < TPS; ++k) {
    const uint32_t w[4] = {raw[k].x, raw[k].y, raw[k].z, raw[k].w};
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += static_cast<double>(__uint_as_float(w[e] << 16));
        acc[2 * e + 1] += static_cast<double>(__uint_as_float(w[e] & 0xffff0000u));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] += static_cast<double>(__uint_as_float(w[e]));
    }
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) part[slot][c * EPC + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    double s = 0.0;
#pragma unroll
    for (int k = 0; k < SLOTS; ++k) s += part[k][threadIdx.x];
    // the exact fp64 sum over the block's tokens, divided once by their count (a power of two, 128,
    // for a full block) and rounded once to fp32
    t.out[(int64_t(bh) * t.out_rows + t.out_off + blk) * D + threadIdx.x] =
        static_cast<float>(s / static_cast<double>(kBlkT * rows * cols));
  }
}

template <typename T, int D>
void launch(const PoolTensor& a, const PoolTensor& b, int heads, const Geom& g, hipStream_t s) {
  if (g.H % kBlkH || g.W % kBlkW) pool_kernel<T, D, true><<<a.wgs + b.wgs, 256, 0, s>>>(a, b, heads, g);
  else pool_kernel<T, D, false><<<a.wgs + b.wgs, 256, 0, s>>>(a, b, heads, g);
}

}  // namespace

lcsa_status pool_k_into(const lcsa_problem* p, const Geom& g, const void* k, lcsa_strides ks, float* out,
                        int32_t out_rows, int32_t out_off, hipStream_t s) {
  PoolTensor tk{k, ks.batch, ks.head, ks.token, out, g.nkb, p->batch * p->heads * g.nkb, out_rows, out_off};
  PoolTensor none{nullptr, 0, 0, 0, nullptr, 1, 0, 1, 0};
  (void)hipGetLastError();
  if (p->dtype == LCSA_BF16) {
    if (p->head_dim == 128) launch<uint16_t, 128>(tk, none, p->heads, g, s);
    else launch<uint16_t, 64>(tk, none, p->heads, g, s);
  } else {
    if (p->head_dim == 128) launch<float, 128>(tk, none, p->heads, g, s);
    else launch<float, 64>(tk, none, p->heads, g, s);
  }
  return hip_status(hipGetLastError(), "pool launch");
}

}  // namespace lcsa

using namespace lcsa;

extern "C" lcsa_status lcsa_pool(const lcsa_problem* p, const void* q, lcsa_strides qs, const void* k,
                                 lcsa_strides ks, float* q_pooled, float* k_pooled, void* stream) {
  Geom g;
  lcsa_status st = validate_problem(p, &g);
  if (st != LCSA_OK) return st;
  if (!q && !k) return fail(LCSA_ERR_INVALID, "lcsa_pool: q and k are both NULL");
  const int64_t hw = int64_t(p->grid_h) * p->grid_w;
  PoolTensor tq{q, qs.batch, qs.head, qs.token, q_pooled, g.nqb, 0, g.nqb, 0};
  PoolTensor tk{k, ks.batch, ks.head, ks.token, k_pooled, g.nkb, 0, g.nkb, 0};
  if (q) {
    if ((st = check_tensor("q", q, qs, p, hw * p->q_frames)) != LCSA_OK) return st;
    if (!q_pooled || reinterpret_cast<uintptr_t>(q_pooled) % 16)
      return fail(LCSA_ERR_INVALID, "q_pooled is NULL or not 16-byte aligned");
    tq.wgs = p->batch * p->heads * g.nqb;
  }
  if (k) {
    if ((st = check_tensor("k", k, ks, p, hw * p->kv_frames)) != LCSA_OK) return st;
    if (!k_pooled || reinterpret_cast<uintptr_t>(k_pooled) % 16)
      return fail(LCSA_ERR_INVALID, "k_pooled is NULL or not 16-byte aligned");
    tk.wgs = p->batch * p->heads * g.nkb;
  }
  const PoolTensor& a = q ? tq : tk;
  const PoolTensor& b = q ? tk : tq;  // when q is NULL, b.wgs == 0
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (p->dtype == LCSA_BF16) {
    if (p->head_dim == 128) launch<uint16_t, 128>(a, b, p->heads, g, s);
    else launch<uint16_t, 64>(a, b, p->heads, g, s);
  } else {
    if (p->head_dim == 128) launch<float, 128>(a, b, p->heads, g, s);
    else launch<float, 64>(a, b, p->heads, g, s);
  }
  return hip_status(hipGetLastError(), "lcsa_pool launch");
}
