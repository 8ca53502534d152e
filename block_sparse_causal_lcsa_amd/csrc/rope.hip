// lcsa_rope_qkv: 3D rotary position embedding of Q and K and the head split of a fused QKV
// projection output, ahead of LCSA in a DiT self-attention layer (FlashVSR summary, sec. 2.2 Stage 1
// names the Wan2.1 DiT; sec. 2.3 discusses its rotary position embeddings at high resolution).
//
// HBM-bound: each lane owns one 16-byte chunk (8 bf16 = 4 rotation pairs) of the head dim of one
// token and a group of head rows, computes the chunk's four angles once and moves that chunk of its
// rows. The angle
// of pair i is pos_axis(i) * freq[i], freq precomputed on the host in fp64 and rounded to fp32;
// sin/cos and the rotation are fp32, the result is rounded once to bf16.
#include <hip/hip_runtime.h>

#include <cmath>

#include "lcsa_internal.h"

namespace lcsa {
namespace {

constexpr int kMaxPairs = 64;  // head_dim <= 128

struct RopeArgs {
  const uint16_t* qkv;
  int64_t qkv_batch, qkv_token;        // elements
  uint16_t* out[3];
  int64_t osb[3], osh[3], ost[3];      // elements
  int32_t heads, head_dim, H, W, frame0;
  int32_t pairs_t, pairs_h;            // pairs rotated by the frame / row position; the rest by column
  int64_t ntok_b;                      // tokens per batch = frames * H * W
  int64_t total;                       // lanes: batch * ntok_b * row groups * head_dim / 8
  float freq[kMaxPairs];
};

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// One lane per (batch, token, group of kRows head rows, 16-byte chunk c of the head dim). The 3*heads
// rows of a token are q of every head, then k, then v; a lane turns chunk c of its q/k rows (the four
// angles depend on the token and c only) and copies chunk c of its v rows. Lanes with consecutive c
// read one head row (d * 2 bytes) together.
constexpr int kRows = 4;

__global__ __launch_bounds__(256) void rope_qkv_kernel(RopeArgs a) {
  const int cpr = a.head_dim / 8;                   // chunks per head row
  const int nrows = 3 * a.heads;
  const int groups = (nrows + kRows - 1) / kRows;
  const int64_t hw = int64_t(a.H) * a.W;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; e < a.total; e += stride) {
    const int64_t tgg = e / cpr;                    // (b * ntok_b + n) * groups + group
    const int c = int(e - tgg * cpr);
    const int64_t tg = tgg / groups;
    const int grp = int(tgg - tg * groups);
    const int64_t b = tg / a.ntok_b, n = tg - b * a.ntok_b;
    const int64_t t = n / hw, sp = n - t * hw;
    const float pos_f = float(a.frame0 + t), pos_h = float(sp / a.W), pos_w = float(sp % a.W);
    float cs[4], sn[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int i = 4 * c + k;                      // pair index: elements 2i, 2i + 1
      const float pos = i < a.pairs_t ? pos_f : (i < a.pairs_t + a.pairs_h ? pos_h : pos_w);
      sincosf(pos * a.freq[i], &sn[k], &cs[k]);
    }
    const uint16_t* row = a.qkv + b * a.qkv_batch + n * a.qkv_token + 8 * c;
    uint4 in[kRows];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int j = grp * kRows + r;
      if (j < nrows) in[r] = *reinterpret_cast<const uint4*>(row + int64_t(j) * a.head_dim);
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int j = grp * kRows + r;
      if (j >= nrows) break;
      const int which = j / a.heads, h = j - which * a.heads;
      uint4 out = in[r];
      if (which < 2) {
        const uint32_t w[4] = {in[r].x, in[r].y, in[r].z, in[r].w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float x0 = bf_lo(w[k]), x1 = bf_hi(w[k]);
          o[k] = bf16_rne(x0 * cs[k] - x1 * sn[k]) | (bf16_rne(x0 * sn[k] + x1 * cs[k]) << 16);
        }
        out = make_uint4(o[0], o[1], o[2], o[3]);
      }
      *reinterpret_cast<uint4*>(a.out[which] + b * a.osb[which] + h * a.osh[which] + n * a.ost[which] + 8 * c) = out;
    }
  }
}

}  // namespace
}  // namespace lcsa

using namespace lcsa;

extern "C" lcsa_status lcsa_rope_qkv(const lcsa_problem* p, const lcsa_rope* rope, const void* qkv, int64_t qkv_batch,
                                     int64_t qkv_token, int32_t frame0, int32_t frames, void* q, lcsa_strides qs,
                                     void* k, lcsa_strides ks, void* v, lcsa_strides vs, void* stream) {
  if (!p) return fail(LCSA_ERR_INVALID, "lcsa_rope_qkv: problem is NULL");
  if (frames < kBlkT || frames % kBlkT)
    return fail(LCSA_ERR_INVALID, "lcsa_rope_qkv: frames %d must be a positive multiple of %d", frames, kBlkT);
  lcsa_problem pc = *p;
  pc.kv_frames = frames;
  pc.q_frame0 = 0;
  pc.q_frames = frames;
  Geom g;
  lcsa_status st = validate_problem(&pc, &g);
  if (st != LCSA_OK) return st;
  if (p->dtype != LCSA_BF16) return fail(LCSA_ERR_UNSUPPORTED, "lcsa_rope_qkv: only bf16 is implemented");
  if (!rope) return fail(LCSA_ERR_INVALID, "lcsa_rope_qkv: rope is NULL");
  if (rope->dim_t < 0 || rope->dim_h < 0 || rope->dim_w < 0 || rope->dim_t % 2 || rope->dim_h % 2 ||
      rope->dim_w % 2 || rope->dim_t + rope->dim_h + rope->dim_w != p->head_dim)
    return fail(LCSA_ERR_INVALID, "lcsa_rope_qkv: dims %d + %d + %d must be even and sum to head_dim %d",
                rope->dim_t, rope->dim_h, rope->dim_w, p->head_dim);
  if (!(rope->theta > 1.0f) || !std::isfinite(rope->theta))
    return fail(LCSA_ERR_INVALID, "lcsa_rope_qkv: theta must be finite and > 1");
  if (frame0 < 0) return fail(LCSA_ERR_INVALID, "lcsa_rope_qkv: frame0 < 0");
  if (!qkv || reinterpret_cast<uintptr_t>(qkv) % 16 || qkv_token < 3 * int64_t(p->heads) * p->head_dim ||
      qkv_token % 8 || qkv_batch % 8 || qkv_batch < 0)
    return fail(LCSA_ERR_INVALID, "lcsa_rope_qkv: qkv NULL, misaligned, or strides that cannot hold a row");
  const int64_t ntok = int64_t(frames) * p->grid_h * p->grid_w;
  if ((st = check_output_tensor("q", q, qs, &pc, ntok)) != LCSA_OK) return st;
  if ((st = check_output_tensor("k", k, ks, &pc, ntok)) != LCSA_OK) return st;
  if ((st = check_output_tensor("v", v, vs, &pc, ntok)) != LCSA_OK) return st;

  RopeArgs a{};
  a.qkv = static_cast<const uint16_t*>(qkv);
  a.qkv_batch = qkv_batch;
  a.qkv_token = qkv_token;
  void* outs[3] = {q, k, v};
  const lcsa_strides ss[3] = {qs, ks, vs};
  for (int i = 0; i < 3; ++i) {
    a.out[i] = static_cast<uint16_t*>(outs[i]);
    a.osb[i] = ss[i].batch;
    a.osh[i] = ss[i].head;
    a.ost[i] = ss[i].token;
  }
  a.heads = p->heads;
  a.head_dim = p->head_dim;
  a.H = p->grid_h;
  a.W = p->grid_w;
  a.frame0 = frame0;
  a.pairs_t = rope->dim_t / 2;
  a.pairs_h = rope->dim_h / 2;
  a.ntok_b = ntok;
  a.total = int64_t(p->batch) * ntok * ((3 * p->heads + kRows - 1) / kRows) * (p->head_dim / 8);
  // freq of pair i within its axis group of dim_axis dims: theta^(-2 i_axis / dim_axis)
  const int dims[3] = {rope->dim_t, rope->dim_h, rope->dim_w};
  int i = 0;
  for (int ax = 0; ax < 3; ++ax)
    for (int j = 0; j < dims[ax] / 2; ++j, ++i)
      a.freq[i] = static_cast<float>(std::pow(static_cast<double>(rope->theta), -2.0 * j / dims[ax]));

  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  const int64_t grid = (a.total + 255) / 256 < 65536 ? (a.total + 255) / 256 : 65536;
  rope_qkv_kernel<<<static_cast<int>(grid), 256, 0, s>>>(a);
  return hip_status(hipGetLastError(), "lcsa_rope_qkv launch");
}
