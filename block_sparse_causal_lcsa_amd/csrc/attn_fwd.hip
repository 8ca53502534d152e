// lcsa_attn_fwd: exact softmax attention of each 128-token query block over the tokens of its kept
// key blocks (FlashVSR summary, sec. 2.2: full attention is applied inside the selected blocks only).
// The kernels are in attn_fwd_impl.h; this unit validates the call and launches the token-window bf16
// variant and the fp32 kernel, attn_fwd_block.hip the block-granular bf16 variants.
#include "attn_fwd_impl.h"

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
  if ((st = check_output_tensor("o", o, os, p, hw * p->q_frames)) != LCSA_OK) return st;
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
  a.div_bpt = make_fastdiv(static_cast<uint32_t>(g.bpt));
  a.div_wb = make_fastdiv(static_cast<uint32_t>(g.Wb));
  a.nrows = p->batch * p->heads * g.nqb;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (p->dtype == LCSA_BF16) {
    a.nwg = a.nrows;  // one query block per workgroup
    const bool ragged = (g.H % kBlkH) != 0 || (g.W % kBlkW) != 0;
    const int mask = token_window(g) ? kMaskWindow : (ragged ? kMaskRagged : kMaskNone);
    if (mask == kMaskWindow) {
      if (p->head_dim == 128) attn_fwd_bf16_kernel<128, kMaskWindow><<<a.nwg, 256, 0, s>>>(a);
      else attn_fwd_bf16_kernel<64, kMaskWindow><<<a.nwg, 256, 0, s>>>(a);
    } else {
      launch_attn_fwd_bf16_block(a, p->head_dim, mask == kMaskRagged, s);
    }
  } else {
    if (p->head_dim == 128) attn_fwd_kernel<float, 128><<<a.nwg, 256, 0, s>>>(a);
    else attn_fwd_kernel<float, 64><<<a.nwg, 256, 0, s>>>(a);
  }
  return hip_status(hipGetLastError(), "lcsa_attn_fwd launch");
}
