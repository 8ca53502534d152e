// Host layer of liblcsa: problem validation, block geometry, K_i rule, CSR layout, errors.
// Pure host C++ (no kernels); built with -ffp-contract=off so the keep-ratio rule is evaluated
// with separately rounded fp64 operations.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "lcsa_internal.h"

namespace lcsa {

namespace {
thread_local std::string g_last_error;
}

lcsa_status fail(lcsa_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

lcsa_status hip_status(int err, const char* what) {
  if (err == 0) return LCSA_OK;
  return fail(LCSA_ERR_HIP, "%s: %s", what, hipGetErrorString(static_cast<hipError_t>(err)));
}

lcsa_status validate_problem(const lcsa_problem* p, Geom* g) {
  if (!p) return fail(LCSA_ERR_INVALID, "problem is NULL");
  if (p->batch < 1 || p->heads < 1) return fail(LCSA_ERR_INVALID, "batch and heads must be >= 1");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(LCSA_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are implemented", p->head_dim);
  if (p->dtype != LCSA_BF16 && p->dtype != LCSA_F32)
    return fail(LCSA_ERR_INVALID, "dtype %d is not an lcsa_dtype", p->dtype);
  if (p->blk_t != kBlkT || p->blk_h != kBlkH || p->blk_w != kBlkW)
    return fail(LCSA_ERR_UNSUPPORTED, "block %dx%dx%d: only 2x8x8 is implemented", p->blk_t, p->blk_h,
                p->blk_w);
  if (p->grid_h < 1 || p->grid_w < 1) return fail(LCSA_ERR_INVALID, "grid must be positive");
  if (p->kv_frames < 1 || p->q_frames < 1 || p->q_frame0 < 0)
    return fail(LCSA_ERR_INVALID, "frame counts must be positive and q_frame0 >= 0");
  if (int64_t(p->q_frame0) + p->q_frames > p->kv_frames)  // 64-bit: the int sum could wrap
    return fail(LCSA_ERR_INVALID, "query frames [%d, %lld) are not inside the %d key frames", p->q_frame0,
                static_cast<long long>(p->q_frame0) + p->q_frames, p->kv_frames);
  if (p->kv_frames % kBlkT || p->q_frames % kBlkT || p->q_frame0 % kBlkT)
    return fail(LCSA_ERR_UNSUPPORTED, "frame counts and q_frame0 must be multiples of %d", kBlkT);
  if (p->win_mode < LCSA_WIN_NONE || p->win_mode > LCSA_WIN_TOKEN_PRESERVING)
    return fail(LCSA_ERR_INVALID, "win_mode %d is not an lcsa_win_mode", p->win_mode);
  if (p->win_mode >= LCSA_WIN_TOKEN_TRUNCATED) {
    if (p->win_h <= 0 || p->win_w <= 0)
      return fail(LCSA_ERR_INVALID, "token window %dx%d must be positive", p->win_h, p->win_w);
  } else if (p->win_mode != LCSA_WIN_NONE) {
    if (p->win_h <= 0 || p->win_w <= 0 || p->win_h % kBlkH || p->win_w % kBlkW ||
        (p->win_h / kBlkH) % 2 == 0 || (p->win_w / kBlkW) % 2 == 0)
      return fail(LCSA_ERR_INVALID, "window %dx%d tokens must be an odd number of 8-token blocks",
                  p->win_h, p->win_w);
  }
  if (p->topk < 0) return fail(LCSA_ERR_INVALID, "topk %d < 0", p->topk);
  if (p->topk == 0 && !(p->keep_ratio > 0.0 && p->keep_ratio <= 1.0))
    return fail(LCSA_ERR_INVALID, "keep_ratio must be in (0, 1] when topk == 0");
  if (!std::isfinite(p->scale) || !(p->scale > 0.0f))
    return fail(LCSA_ERR_INVALID, "scale must be finite and positive");

  const int64_t hw = static_cast<int64_t>(p->grid_h) * p->grid_w;
  const int64_t nk_tok = hw * p->kv_frames;
  // edge blocks of a grid that is not a multiple of 8 are partial (fewer rows or columns)
  const int64_t hb_n = (int64_t(p->grid_h) + kBlkH - 1) / kBlkH, wb_n = (int64_t(p->grid_w) + kBlkW - 1) / kBlkW;
  const int64_t bpt = hb_n * wb_n;
  const int64_t nkb = bpt * (p->kv_frames / kBlkT);
  // every kernel indexes blocks, rows and (batch, head) pairs with 32-bit integers
  if (nk_tok > (int64_t(1) << 30) || nkb * p->batch * p->heads > (int64_t(1) << 30))
    return fail(LCSA_ERR_UNSUPPORTED, "problem too large for 32-bit block indexing");
  if (g) {
    g->H = p->grid_h;
    g->W = p->grid_w;
    g->Hb = static_cast<int32_t>(hb_n);
    g->Wb = static_cast<int32_t>(wb_n);
    g->bpt = static_cast<int32_t>(bpt);
    g->nqb = static_cast<int32_t>(bpt * (p->q_frames / kBlkT));
    g->nkb = static_cast<int32_t>(nkb);
    g->q_tb0 = p->q_frame0 / kBlkT;
    g->win_mode = p->win_mode;
    const bool blockwin = p->win_mode == LCSA_WIN_TRUNCATED || p->win_mode == LCSA_WIN_PRESERVING;
    g->wbh = blockwin ? p->win_h / kBlkH : 0;
    g->wbw = blockwin ? p->win_w / kBlkW : 0;
    g->wth = blockwin || p->win_mode == LCSA_WIN_NONE ? 0 : p->win_h;
    g->wtw = blockwin || p->win_mode == LCSA_WIN_NONE ? 0 : p->win_w;
  }
  return LCSA_OK;
}

int keep_count(const lcsa_problem* p, int n) {
  if (p->topk > 0) return p->topk < n ? p->topk : n;
  double x = p->keep_ratio * static_cast<double>(n);
  x = x + 0.5;
  double k = std::floor(x);
  if (k < 1.0) k = 1.0;
  if (k > n) k = n;
  return static_cast<int>(k);
}

lcsa_status check_tensor(const char* name, const void* ptr, lcsa_strides s, const lcsa_problem* p,
                         int64_t ntok) {
  if (!ptr) return fail(LCSA_ERR_INVALID, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(ptr) % 16)
    return fail(LCSA_ERR_INVALID, "%s is not 16-byte aligned", name);
  const int64_t vec = 16 / dtype_size(p);  // elements per 16 bytes
  if (s.batch < 0 || s.head < 0 || s.token < p->head_dim)
    return fail(LCSA_ERR_INVALID, "%s strides (%lld, %lld, %lld) cannot hold [.., %d] rows", name,
                (long long)s.batch, (long long)s.head, (long long)s.token, p->head_dim);
  if (s.batch % vec || s.head % vec || s.token % vec)
    return fail(LCSA_ERR_INVALID, "%s strides must be multiples of 16 bytes", name);
  if (ntok < 1) return fail(LCSA_ERR_INVALID, "%s has no tokens", name);
  return LCSA_OK;
}

lcsa_status check_output_tensor(const char* name, void* ptr, lcsa_strides s, const lcsa_problem* p,
                                int64_t ntok) {
  lcsa_status st = check_tensor(name, ptr, s, p, ntok);
  if (st != LCSA_OK) return st;
  // Every element (b, h, t, c) must have its own address, or two workgroups would write the same
  // memory. Sort the dimensions of extent > 1 by stride; each stride must step past everything the
  // smaller dimensions reach.
  struct Dim { int64_t stride, extent; } d[4] = {
      {s.batch, p->batch}, {s.head, p->heads}, {s.token, ntok}, {1, p->head_dim}};
  for (int i = 1; i < 4; ++i)
    for (int j = i; j > 0 && d[j].stride < d[j - 1].stride; --j) {
      const Dim t = d[j]; d[j] = d[j - 1]; d[j - 1] = t;
    }
  int64_t reach = 0;  // largest offset reached by the dimensions already visited
  for (int i = 0; i < 4; ++i) {
    if (d[i].extent <= 1) continue;
    if (d[i].stride <= reach)
      return fail(LCSA_ERR_INVALID, "%s strides (%lld, %lld, %lld) make output rows overlap", name,
                  (long long)s.batch, (long long)s.head, (long long)s.token);
    reach += (d[i].extent - 1) * d[i].stride;
  }
  return LCSA_OK;
}

}  // namespace lcsa

using namespace lcsa;

extern "C" {

lcsa_status lcsa_csr_layout(const lcsa_problem* p, int32_t* nqb, int32_t* nkb, int32_t* nnz_per_head,
                            int32_t* row_ptr_host) {
  Geom g;
  lcsa_status st = validate_problem(p, &g);
  if (st != LCSA_OK) return st;
  int64_t acc = 0;
  for (int i = 0; i < g.nqb; ++i) {
    if (row_ptr_host) row_ptr_host[i] = static_cast<int32_t>(acc);
    acc += keep_count(p, n_visible(g, i));
  }
  if (acc > INT32_MAX) return fail(LCSA_ERR_UNSUPPORTED, "more than 2^31 kept blocks per head");
  if (row_ptr_host) row_ptr_host[g.nqb] = static_cast<int32_t>(acc);
  if (nqb) *nqb = g.nqb;
  if (nkb) *nkb = g.nkb;
  if (nnz_per_head) *nnz_per_head = static_cast<int32_t>(acc);
  return LCSA_OK;
}

const char* lcsa_status_string(lcsa_status s) {
  switch (s) {
    case LCSA_OK: return "LCSA_OK";
    case LCSA_ERR_INVALID: return "LCSA_ERR_INVALID";
    case LCSA_ERR_UNSUPPORTED: return "LCSA_ERR_UNSUPPORTED";
    case LCSA_ERR_HIP: return "LCSA_ERR_HIP";
  }
  return "unknown lcsa_status";
}

const char* lcsa_last_error(void) { return g_last_error.c_str(); }

int32_t lcsa_version(void) { return 100; }  // 0.1.0

}  // extern "C"
