// Streaming state for chunk-by-chunk LCSA (lcsa_stream_*): K/V rings holding the newest temporal
// blocks and the pooled K of those blocks, so that each chunk moves and pools only its own block
// (FlashVSR summary, sec. 2.2 Stage 3, the KV cache; sec. 3, one temporal block per chunk).
//
// Device layout inside the caller's memory, per (batch, head), C = cache_tblocks, R = ring_tblocks,
// T = tokens of one temporal block (2 * H * W):
//   K ring, V ring: R slots of T tokens x d, dtype of the problem, filled in order. The held blocks
//                   are slots [wpos - held, wpos): the window is one view with the ring's strides.
//                   When wpos reaches R, the newest C - 1 blocks are copied to slots [0, C - 1)
//                   (R >= 2C - 1 keeps source and destination apart), once every R - C + 2 pushes.
//   pooled K:       two buffers of C * (blocks per temporal block) rows x d fp32, used alternately.
//                   After a push the current buffer holds the held blocks' means contiguously
//                   ([B, Hh, held * bpt, d]), the layout lcsa_score_select takes.
// A push is at most one copy kernel (the new K and V into their slot unless the producer wrote them
// there, and the kept pooled rows shifted into the other buffer) and one pooling launch of the new
// K straight into that buffer.
#include <hip/hip_runtime.h>

#include "lcsa_internal.h"

namespace lcsa {
namespace {

struct StreamLayout {
  size_t k_ring, v_ring, kbar0, kbar1, total;
  int64_t tb_tokens;   // tokens per temporal block
  int64_t ring_head;   // elements per (batch, head) in a ring
  int64_t kbar_rows;   // rows per (batch, head) in a pooled-K buffer at capacity
};

StreamLayout stream_layout(const lcsa_problem* p, const Geom& g, int32_t cap, int32_t ring) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  StreamLayout l{};
  const size_t bh = size_t(p->batch) * p->heads;
  l.tb_tokens = int64_t(kBlkT) * p->grid_h * p->grid_w;
  l.ring_head = int64_t(ring) * l.tb_tokens * p->head_dim;
  l.kbar_rows = int64_t(cap) * g.bpt;
  const size_t rbytes = bh * size_t(l.ring_head) * dtype_size(p);
  const size_t kbar = bh * size_t(l.kbar_rows) * p->head_dim * sizeof(float);
  l.k_ring = 0;
  l.v_ring = up(rbytes);
  l.kbar0 = l.v_ring + up(rbytes);
  l.kbar1 = l.kbar0 + up(kbar);
  l.total = l.kbar1 + up(kbar);
  return l;
}

// Checks the chunk problem (a valid problem whose queries are one temporal block) and the cache and
// ring sizes; fills the one-block problem and its geometry.
lcsa_status check_chunk(const lcsa_problem* chunk, int32_t cap, int32_t ring, lcsa_problem* win1, Geom* g) {
  if (!chunk) return fail(LCSA_ERR_INVALID, "lcsa_stream: chunk problem is NULL");
  if (cap < 1 || cap > 4096) return fail(LCSA_ERR_INVALID, "lcsa_stream: cache_tblocks %d outside [1, 4096]", cap);
  const int32_t min_ring = cap > 1 ? 2 * cap - 1 : 1;
  if (ring < min_ring || ring > 65536)
    return fail(LCSA_ERR_INVALID, "lcsa_stream: ring_tblocks %d, must be in [%d, 65536]", ring, min_ring);
  if (chunk->q_frames != kBlkT)
    return fail(LCSA_ERR_UNSUPPORTED, "lcsa_stream: chunks of %d query frames; one temporal block (%d) is implemented",
                chunk->q_frames, kBlkT);
  *win1 = *chunk;
  win1->kv_frames = kBlkT;  // geometry of one block; validates everything else
  win1->q_frame0 = 0;
  return validate_problem(win1, g);
}

// Copies n_tok tokens x cpt 16-byte chunks per (batch, head) from src (strides in chunks) to
// dst (ring layout: ring_head chunks per (batch, head), contiguous tokens) for K and V together.
struct CopyArgs {
  const uint4* k_src;
  const uint4* v_src;
  int64_t ksb, ksh, kst, vsb, vsh, vst;
  uint4* k_dst;
  uint4* v_dst;
  int64_t ring_head;
  int64_t dst_tok0;   // first destination token in the ring
  int32_t heads, cpt;
  int32_t lcpt;       // log2(cpt): cpt = head_dim * element size / 16 is 8, 16 or 32
  int64_t bh_n;       // B * Hh
  int64_t n_tok;
  int64_t n;          // B * Hh * n_tok * cpt
};

// Shifts the kept pooled rows into the other buffer: new[bh][r] = old[bh][r + shift], r < keep.
struct ShiftArgs {
  const float4* old_buf;
  float4* new_buf;
  int32_t old_rows, new_rows, keep_rows, shift_rows, vpr;
  int64_t n;          // B * Hh * keep_rows * vpr
};

// K/V copy: blockIdx.x tiles the tokens (256 / cpt per workgroup), blockIdx.y walks the (batch,
// head) pairs, so a lane's token and 16-byte chunk come from shifts and no division runs per chunk.
// The pooled-K shift is a grid-stride loop over the whole grid.
__global__ __launch_bounds__(256) void stream_copy_kernel(CopyArgs c, ShiftArgs s) {
  if (c.n > 0) {
    const int64_t tok = int64_t(blockIdx.x) * (256 >> c.lcpt) + (threadIdx.x >> c.lcpt);
    const int64_t ch = threadIdx.x & ((1 << c.lcpt) - 1);
    if (tok < c.n_tok) {
      for (int64_t bh = blockIdx.y; bh < c.bh_n; bh += gridDim.y) {
        const int64_t b = bh / c.heads, h = bh - b * c.heads;
        const int64_t dst = bh * c.ring_head + ((c.dst_tok0 + tok) << c.lcpt) + ch;
        c.k_dst[dst] = c.k_src[b * c.ksb + h * c.ksh + tok * c.kst + ch];
        c.v_dst[dst] = c.v_src[b * c.vsb + h * c.vsh + tok * c.vst + ch];
      }
    }
  }
  const int64_t stride = int64_t(gridDim.x) * gridDim.y * blockDim.x;
  for (int64_t e = (int64_t(blockIdx.y) * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x; e < s.n; e += stride) {
    const int64_t ch = e % s.vpr, r = (e / s.vpr) % s.keep_rows, bh = e / (int64_t(s.vpr) * s.keep_rows);
    s.new_buf[(bh * s.new_rows + r) * s.vpr + ch] = s.old_buf[(bh * s.old_rows + r + s.shift_rows) * s.vpr + ch];
  }
}

lcsa_status launch_copy(const CopyArgs& c, const ShiftArgs& s, hipStream_t hs, const char* what) {
  if (c.n == 0 && s.n == 0) return LCSA_OK;
  dim3 grid(1, 1);
  if (c.n > 0) {
    if (c.cpt != (1 << c.lcpt) || c.lcpt < 3 || c.lcpt > 5) return fail(LCSA_ERR_UNSUPPORTED, "%s: chunk count", what);
    const int64_t tpb = 256 >> c.lcpt;
    grid.x = static_cast<uint32_t>((c.n_tok + tpb - 1) / tpb);
    grid.y = static_cast<uint32_t>(c.bh_n < 65535 ? c.bh_n : 65535);
  } else {
    grid.x = static_cast<uint32_t>((s.n + 255) / 256 < 8192 ? (s.n + 255) / 256 : 8192);
  }
  (void)hipGetLastError();
  stream_copy_kernel<<<grid, 256, 0, hs>>>(c, s);
  return hip_status(hipGetLastError(), what);
}

lcsa_status check_state(const lcsa_stream* s, lcsa_problem* w1, Geom* g, StreamLayout* l) {
  if (!s) return fail(LCSA_ERR_INVALID, "lcsa_stream: state is NULL");
  lcsa_status st = check_chunk(&s->chunk, s->cache_tblocks, s->ring_tblocks, w1, g);
  if (st != LCSA_OK) return st;
  *l = stream_layout(&s->chunk, *g, s->cache_tblocks, s->ring_tblocks);
  // wpos = held - 1 only between a compacting reserve and the push that follows it
  if (!s->mem || s->mem_bytes < l->total || s->held < 0 || s->held > s->cache_tblocks || s->pushed < s->held ||
      s->wpos < s->held - 1 || s->wpos < 0 || s->wpos > s->ring_tblocks)
    return fail(LCSA_ERR_INVALID, "lcsa_stream: state not initialised by lcsa_stream_init");
  return LCSA_OK;
}

int64_t elem_bytes(const lcsa_problem* p) { return dtype_size(p); }

// Makes room for the next block: when the write position is at the end of the ring, copies the
// newest min(held, C - 1) blocks to the front.
lcsa_status make_room(lcsa_stream* s, const lcsa_problem& w1, const StreamLayout& l, hipStream_t hs) {
  if (s->wpos < s->ring_tblocks) return LCSA_OK;
  const int keep = s->held < s->cache_tblocks - 1 ? s->held : s->cache_tblocks - 1;
  if (keep > 0) {
    const int epc = 16 / dtype_size(&w1);
    char* mem = static_cast<char*>(s->mem);
    const int64_t cpt = w1.head_dim / epc, rh = l.ring_head / epc;
    const int64_t src_tok0 = int64_t(s->wpos - keep) * l.tb_tokens;
    CopyArgs c{};
    c.k_src = reinterpret_cast<const uint4*>(mem + l.k_ring) + src_tok0 * cpt;
    c.v_src = reinterpret_cast<const uint4*>(mem + l.v_ring) + src_tok0 * cpt;
    c.ksb = int64_t(w1.heads) * rh; c.ksh = rh; c.kst = cpt;
    c.vsb = c.ksb; c.vsh = rh; c.vst = cpt;
    c.k_dst = reinterpret_cast<uint4*>(mem + l.k_ring);
    c.v_dst = reinterpret_cast<uint4*>(mem + l.v_ring);
    c.ring_head = rh;
    c.dst_tok0 = 0;
    c.heads = w1.heads;
    c.cpt = static_cast<int32_t>(cpt);
    c.lcpt = __builtin_ctz(static_cast<unsigned>(cpt));
    c.bh_n = int64_t(w1.batch) * w1.heads;
    c.n_tok = int64_t(keep) * l.tb_tokens;
    c.n = int64_t(w1.batch) * w1.heads * c.n_tok * cpt;
    ShiftArgs none{};
    const lcsa_status st = launch_copy(c, none, hs, "lcsa_stream compaction launch");
    if (st != LCSA_OK) return st;
  }
  s->wpos = keep;
  return LCSA_OK;
}

}  // namespace
}  // namespace lcsa

using namespace lcsa;

extern "C" lcsa_status lcsa_stream_state_size(const lcsa_problem* chunk, int32_t cache_tblocks, int32_t ring_tblocks,
                                              size_t* bytes) {
  lcsa_problem w1;
  Geom g;
  lcsa_status st = check_chunk(chunk, cache_tblocks, ring_tblocks, &w1, &g);
  if (st != LCSA_OK) return st;
  if (!bytes) return fail(LCSA_ERR_INVALID, "lcsa_stream_state_size: bytes is NULL");
  *bytes = stream_layout(chunk, g, cache_tblocks, ring_tblocks).total;
  return LCSA_OK;
}

extern "C" lcsa_status lcsa_stream_init(lcsa_stream* s, const lcsa_problem* chunk, int32_t cache_tblocks,
                                        int32_t ring_tblocks, void* mem, size_t mem_bytes) {
  lcsa_problem w1;
  Geom g;
  lcsa_status st = check_chunk(chunk, cache_tblocks, ring_tblocks, &w1, &g);
  if (st != LCSA_OK) return st;
  if (!s) return fail(LCSA_ERR_INVALID, "lcsa_stream_init: state is NULL");
  if (!mem || reinterpret_cast<uintptr_t>(mem) % 256)
    return fail(LCSA_ERR_INVALID, "lcsa_stream_init: mem is NULL or not 256-byte aligned");
  const size_t need = stream_layout(chunk, g, cache_tblocks, ring_tblocks).total;
  if (mem_bytes < need)
    return fail(LCSA_ERR_INVALID, "lcsa_stream_init: %zu bytes of state memory, %zu needed", mem_bytes, need);
  s->chunk = *chunk;
  s->cache_tblocks = cache_tblocks;
  s->ring_tblocks = ring_tblocks;
  s->held = 0;
  s->wpos = 0;
  s->pushed = 0;
  s->mem = mem;
  s->mem_bytes = mem_bytes;
  return LCSA_OK;
}

extern "C" lcsa_status lcsa_stream_reserve(lcsa_stream* s, void** k_slot, lcsa_strides* ks, void** v_slot,
                                           lcsa_strides* vs, void* stream) {
  lcsa_problem w1;
  Geom g;
  StreamLayout l;
  lcsa_status st = check_state(s, &w1, &g, &l);
  if (st != LCSA_OK) return st;
  if ((st = make_room(s, w1, l, static_cast<hipStream_t>(stream))) != LCSA_OK) return st;
  char* mem = static_cast<char*>(s->mem);
  const int64_t off = int64_t(s->wpos) * l.tb_tokens * w1.head_dim * elem_bytes(&w1);
  const lcsa_strides rs{int64_t(w1.heads) * l.ring_head, l.ring_head, w1.head_dim};
  if (k_slot) *k_slot = mem + l.k_ring + off;
  if (v_slot) *v_slot = mem + l.v_ring + off;
  if (ks) *ks = rs;
  if (vs) *vs = rs;
  return LCSA_OK;
}

extern "C" lcsa_status lcsa_stream_push(lcsa_stream* s, const void* k_new, lcsa_strides ks, const void* v_new,
                                        lcsa_strides vs, void* stream) {
  lcsa_problem w1;
  Geom g;
  StreamLayout l;
  lcsa_status st = check_state(s, &w1, &g, &l);
  if (st != LCSA_OK) return st;
  if ((st = check_tensor("k_new", k_new, ks, &w1, l.tb_tokens)) != LCSA_OK) return st;
  if ((st = check_tensor("v_new", v_new, vs, &w1, l.tb_tokens)) != LCSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  void* k_slot = nullptr;
  void* v_slot = nullptr;
  lcsa_strides rs{};
  if ((st = lcsa_stream_reserve(s, &k_slot, &rs, &v_slot, nullptr, stream)) != LCSA_OK) return st;
  const bool in_place = k_new == k_slot && v_new == v_slot && ks.batch == rs.batch && ks.head == rs.head &&
                        ks.token == rs.token && vs.batch == rs.batch && vs.head == rs.head && vs.token == rs.token;
  const int cap = s->cache_tblocks;
  const int old_held = s->held, new_held = old_held < cap ? old_held + 1 : cap;
  const int epc = 16 / dtype_size(&w1);
  char* mem = static_cast<char*>(s->mem);
  // the pooled-K buffer that receives this push: buffers alternate, pushed even -> buffer 0
  float* kb_old = reinterpret_cast<float*>(mem + ((s->pushed & 1) ? l.kbar0 : l.kbar1));
  float* kb_new = reinterpret_cast<float*>(mem + ((s->pushed & 1) ? l.kbar1 : l.kbar0));
  const int64_t bh = int64_t(w1.batch) * w1.heads;

  CopyArgs c{};
  if (!in_place) {
    c.k_src = static_cast<const uint4*>(k_new);
    c.v_src = static_cast<const uint4*>(v_new);
    c.ksb = ks.batch / epc; c.ksh = ks.head / epc; c.kst = ks.token / epc;
    c.vsb = vs.batch / epc; c.vsh = vs.head / epc; c.vst = vs.token / epc;
    c.k_dst = reinterpret_cast<uint4*>(mem + l.k_ring);
    c.v_dst = reinterpret_cast<uint4*>(mem + l.v_ring);
    c.ring_head = l.ring_head / epc;
    c.dst_tok0 = int64_t(s->wpos) * l.tb_tokens;
    c.heads = w1.heads;
    c.cpt = w1.head_dim / epc;
    c.lcpt = __builtin_ctz(static_cast<unsigned>(c.cpt));
    c.bh_n = bh;
    c.n_tok = l.tb_tokens;
    c.n = bh * l.tb_tokens * c.cpt;
  }
  ShiftArgs sh{};
  sh.old_buf = reinterpret_cast<const float4*>(kb_old);
  sh.new_buf = reinterpret_cast<float4*>(kb_new);
  sh.vpr = w1.head_dim / 4;
  sh.old_rows = old_held * g.bpt;
  sh.new_rows = new_held * g.bpt;
  sh.keep_rows = (new_held - 1) * g.bpt;
  sh.shift_rows = (old_held - (new_held - 1)) * g.bpt;
  sh.n = bh * sh.keep_rows * sh.vpr;
  if ((st = launch_copy(c, sh, hs, "lcsa_stream_push copy launch")) != LCSA_OK) return st;
  // pooled K of the new block into rows [(new_held - 1) * bpt, new_held * bpt) of kb_new
  if ((st = pool_k_into(&w1, g, k_new, ks, kb_new, sh.new_rows, sh.keep_rows, hs)) != LCSA_OK) return st;
  s->held = new_held;
  s->wpos += 1;
  s->pushed += 1;
  return LCSA_OK;
}

extern "C" lcsa_status lcsa_stream_window(const lcsa_stream* s, lcsa_problem* window, const void** k,
                                          lcsa_strides* ks, const void** v, lcsa_strides* vs,
                                          const float** k_pooled) {
  lcsa_problem w1;
  Geom g;
  StreamLayout l;
  lcsa_status st = check_state(s, &w1, &g, &l);
  if (st != LCSA_OK) return st;
  if (s->held < 1) return fail(LCSA_ERR_INVALID, "lcsa_stream_window: nothing pushed yet");
  if (s->wpos < s->held)
    return fail(LCSA_ERR_INVALID, "lcsa_stream_window: the ring was compacted by lcsa_stream_reserve; push first");
  const int w = s->held;
  const int64_t off = int64_t(s->wpos - w) * l.tb_tokens * w1.head_dim * elem_bytes(&w1);
  const char* mem = static_cast<const char*>(s->mem);
  if (window) {
    *window = s->chunk;
    window->kv_frames = kBlkT * w;
    window->q_frame0 = kBlkT * (w - 1);
    window->q_frames = kBlkT;
  }
  const lcsa_strides rs{int64_t(w1.heads) * l.ring_head, l.ring_head, w1.head_dim};
  if (k) *k = mem + l.k_ring + off;
  if (v) *v = mem + l.v_ring + off;
  if (ks) *ks = rs;
  if (vs) *vs = rs;
  // the buffer written by the last push: pushed odd -> buffer 0
  if (k_pooled) *k_pooled = reinterpret_cast<const float*>(mem + ((s->pushed & 1) ? l.kbar0 : l.kbar1));
  return LCSA_OK;
}
