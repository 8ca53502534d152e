/*
 * lcsa.h - C ABI of liblcsa.so: locality-constrained block-sparse causal attention (LCSA)
 * forward and backward on AMD MI355X (gfx950).
 *
 * The operation is the one described for FlashVSR's stage-2 sparse-causal attention and its
 * locality-constrained inference ("FlashVSR: Towards Real-time Diffusion-Based Streaming Video
 * Super Resolution", fmread pdfshare summary, sec. 2.2 "Stage 2: block-sparse causal attention
 * adaptation" and sec. 2.3 "locality-constrained sparse attention"):
 *   1. Q and K are cut into non-overlapping spatio-temporal blocks of blk_t x blk_h x blk_w tokens
 *      (2x8x8) and each block is average-pooled to one feature vector      -> lcsa_pool
 *   2. a coarse block-to-block map s_ij = scale * <qbar_i, kbar_j> is scored over the key blocks
 *      that query block i may see (latent-frame causality, optional local spatial window), and the
 *      Top-K key blocks of every query block are kept                       -> lcsa_score_select
 *   3. exact softmax attention runs over the tokens of the kept blocks only -> lcsa_attn_fwd
 *
 * Conventions shared by every entry point:
 *   - Tensors are caller-owned device memory (hipMalloc / torch), the library allocates nothing.
 *   - Token tensors are [batch, heads, tokens, head_dim] with element strides given by
 *     lcsa_strides; the head_dim stride is 1. Tokens are in raster order n = (t*H + h)*W + w,
 *     t counted from the tensor's first latent frame. Base pointers must be 16-byte aligned and
 *     the batch/head/token strides multiples of 8 elements (16 bytes).
 *   - Every device call is asynchronous on `stream` (a hipStream_t; NULL = the null stream) and
 *     never synchronises the host. Validation is synchronous and happens before any launch: an
 *     invalid problem returns LCSA_ERR_INVALID / LCSA_ERR_UNSUPPORTED and launches nothing. A failed
 *     launch returns LCSA_ERR_HIP. A device fault surfaces at the caller's next synchronisation.
 *   - lcsa_last_error() gives a thread-local message for the last non-OK return of this thread.
 *   - Inputs must be finite. All calls are stateless and re-entrant.
 */
#ifndef LCSA_H_
#define LCSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LCSA_OK = 0,
  LCSA_ERR_INVALID = 1,      /* inconsistent sizes, null or misaligned pointer, bad stride */
  LCSA_ERR_UNSUPPORTED = 2,  /* a valid problem outside what the kernels implement */
  LCSA_ERR_HIP = 3           /* a HIP runtime call or kernel launch failed */
} lcsa_status;

typedef enum { LCSA_BF16 = 0, LCSA_F32 = 1 } lcsa_dtype;

/* Locality window rules (sec. 2.3 and the sec. 3 ablation name two: boundary-truncated and
 * boundary-preserving). The window is block-granular and spatial: w_b = win/blk blocks per axis
 * (odd), r = (w_b-1)/2. TRUNCATED keeps the blocks within r of the query block, cut at the frame
 * edge; PRESERVING slides a w_b-wide window inward at the edge (start = clamp(c-r, 0, N-w_b)), so
 * every query keeps w_b blocks per axis. The same window applies in every visible temporal block. */
/* TOKEN_TRUNCATED / TOKEN_PRESERVING: the same two rules per query token instead of per block. A query
 * token at (h, w) sees the key tokens in rows [h - (win_h-1)/2, h - (win_h-1)/2 + win_h - 1] and the
 * like columns (win_h, win_w any positive token counts), cut at the frame edge or shifted inside. A
 * key block is a candidate of query block i when some token of i sees some token of it; inside a kept
 * block only the tokens in the query token's window take part. A query token that sees no token of
 * its kept blocks gets O = 0 and lse = -inf. */
typedef enum {
  LCSA_WIN_NONE = 0,
  LCSA_WIN_TRUNCATED = 1,
  LCSA_WIN_PRESERVING = 2,
  LCSA_WIN_TOKEN_TRUNCATED = 3,
  LCSA_WIN_TOKEN_PRESERVING = 4
} lcsa_win_mode;

typedef struct {
  int32_t batch, heads, head_dim;  /* head_dim in {64, 128} */
  int32_t grid_h, grid_w;          /* latent tokens per frame (>= 1). Blocks are cut from the origin;
                                      when not a multiple of 8, the last block row / column is partial */
  int32_t kv_frames;               /* K/V hold latent frames [0, kv_frames) */
  int32_t q_frame0, q_frames;      /* Q holds latent frames [q_frame0, q_frame0 + q_frames) */
  int32_t blk_t, blk_h, blk_w;     /* block shape in tokens; only 2 x 8 x 8 is implemented */
  int32_t win_mode;                /* lcsa_win_mode */
  int32_t win_h, win_w;            /* window in tokens; block modes: win/blk must be an odd integer */
  int32_t topk;                    /* > 0: K_i = min(topk, n_i); 0: K_i from keep_ratio */
  double keep_ratio;               /* (0, 1]: K_i = clamp(floor(keep_ratio * n_i + 0.5), 1, n_i) */
  float scale;                     /* softmax / block-score scale (> 0), e.g. 1/sqrt(head_dim) */
  int32_t dtype;                   /* lcsa_dtype of Q, K, V and O */
} lcsa_problem;

typedef struct { int64_t batch, head, token; } lcsa_strides; /* in elements */

/* Geometry and CSR layout of the selection (host only, pure, no device work).
 * Query block i covers the tokens of temporal block tb_i = (q_frame0 + 2*(i / (Hb*Wb))) / blk_t,
 * block row hb and block column wb, i = (tb_rel*Hb + hb)*Wb + wb; key block j likewise from frame 0.
 * Key block j is visible from i iff tb_j <= tb_i (causal masking, sec. 2.2) and it lies in i's
 * window on both axes (sec. 2.3); n_i counts them. row_ptr = exclusive prefix sum of K_i; it is the
 * same for every (batch, head).
 * Outputs (any may be NULL): *nqb, *nkb block counts; *nnz_per_head = row_ptr[nqb];
 * row_ptr_host, if non-NULL, receives nqb + 1 int32 entries (call first with NULL to size it). */
lcsa_status lcsa_csr_layout(const lcsa_problem* p, int32_t* nqb, int32_t* nkb,
                            int32_t* nnz_per_head, int32_t* row_ptr_host);

/* Block mean pooling (sec. 2.2: average pooling of Q and K over each block).
 * q: [B, Hh, q_frames*H*W, d] (dtype), k: [B, Hh, kv_frames*H*W, d] (dtype).
 * q_pooled: [B, Hh, nqb, d] fp32 contiguous; k_pooled: [B, Hh, nkb, d] fp32 contiguous.
 * Each output is the mean of the block's 128 tokens (fewer in a partial edge block: the tokens
 * inside the grid), accumulated in fp64, rounded once to fp32.
 * q (with q_pooled) or k (with k_pooled) may be NULL to pool only the other tensor. */
lcsa_status lcsa_pool(const lcsa_problem* p, const void* q, lcsa_strides qs, const void* k,
                      lcsa_strides ks, float* q_pooled, float* k_pooled, void* stream);

/* Coarse block map, masks and per-row Top-K (sec. 2.2 "coarse block attention map ... Top-K block
 * pairs"; sec. 2.3 window). For every (b, h, i): s_ij = scale * <q_pooled_i, k_pooled_j> in fp64
 * over the visible j; keeps the K_i = row_ptr[i+1] - row_ptr[i] largest, exact ties to the lower j.
 * row_ptr: device int32 [nqb + 1] as produced by lcsa_csr_layout.
 * col_idx: device int32 [B, Hh, nnz_per_head]; row i's kept key blocks at
 *          [row_ptr[i], row_ptr[i+1]) in ascending order.
 * scores_dbg: NULL, or device fp64 [B, Hh, nqb, nkb] receiving s_ij (-inf where not visible). */
lcsa_status lcsa_score_select(const lcsa_problem* p, const float* q_pooled, const float* k_pooled,
                              const int32_t* row_ptr, int32_t* col_idx, double* scores_dbg,
                              void* stream);

/* Exact attention over the kept blocks (sec. 2.2 "full attention inside the selected blocks").
 * For each query token of block i: O = softmax(scale * q K_S^T) V_S over all tokens of the blocks
 * S = col_idx[b, h, row_ptr[i]:row_ptr[i+1]] (no token mask inside a kept block; a kept block is
 * always fully visible under block causality and a block-granular window). In a partial edge block
 * only the tokens inside the grid exist: they alone are keys, and only they get O and lse.
 * q: [B, Hh, Nq, d]; k, v: [B, Hh, Nk, d]; o: [B, Hh, Nq, d], all of the problem's dtype.
 * lse: NULL, or device fp32 [B, Hh, Nq] contiguous: natural log of the softmax denominator.
 * Arithmetic: bf16 inputs as given (fp32 inputs are rounded to bf16 on load), bf16 MFMA with fp32
 * accumulation for QK^T and PV, online softmax in fp32, P rounded to bf16 for PV while the
 * denominator (and lse) sums the fp32 P; O written as bf16 (RNE) or fp32. col_idx entries outside
 * [0, nkb) are skipped. */
lcsa_status lcsa_attn_fwd(const lcsa_problem* p, const void* q, lcsa_strides qs, const void* k,
                          lcsa_strides ks, const void* v, lcsa_strides vs, const int32_t* row_ptr,
                          const int32_t* col_idx, void* o, lcsa_strides os, float* lse,
                          void* stream);

/* Gradients of lcsa_attn_fwd for a fixed selection (training the sparse-causal model, sec. 2.2
 * "Stage 2": the attention is trained block-sparse; the Top-K selection itself is not
 * differentiated). With P = softmax(scale * q K_S^T) over the kept blocks S of each query token's
 * block and upstream gradient dO:
 *   Delta = rowsum(dO * O); dP = dO V_S^T; dS = P * (dP - Delta)
 *   dQ = scale * dS K_S;  dK_S += scale * dS^T Q;  dV_S += P^T dO
 * dK and dV of a key block sum over every query block that kept it; key blocks nobody kept get 0.
 * q, k, v, o, d_o: bf16 [B, Hh, N, d] with lcsa_strides (o, lse: the forward's outputs for the same
 *   q, k, v and selection; d_o: dL/dO). row_ptr, col_idx: the selection, as lcsa_score_select
 *   writes it (rows strictly ascending; entries outside [0, nkb) are skipped).
 * dq: fp32 [B, Hh, Nq, d], dk, dv: fp32 [B, Hh, Nk, d], contiguous, 16-byte aligned, fully written.
 * workspace: device memory of lcsa_attn_bwd_workspace_size bytes, 256-byte aligned, caller-owned,
 *   no initial contents required; it must not be shared by calls that overlap in time.
 * Arithmetic: bf16 MFMA with fp32 accumulation; P and dS rounded to bf16 for the dV, dK and dQ
 * products; Delta in fp32 from the bf16 O. Deterministic: no atomics on the gradients.
 * Partial edge blocks (grids that are not multiples of 8) hold only the tokens inside the grid, as in
 * lcsa_attn_fwd. Only bf16 problems are implemented (LCSA_ERR_UNSUPPORTED otherwise). */
lcsa_status lcsa_attn_bwd_workspace_size(const lcsa_problem* p, size_t* bytes);
lcsa_status lcsa_attn_bwd(const lcsa_problem* p, const void* q, lcsa_strides qs, const void* k,
                          lcsa_strides ks, const void* v, lcsa_strides vs, const void* o,
                          lcsa_strides os, const void* d_o, lcsa_strides dos, const float* lse,
                          const int32_t* row_ptr, const int32_t* col_idx, float* dq, float* dk,
                          float* dv, void* workspace, size_t workspace_bytes, void* stream);

/* lcsa_attn_bwd without a caller workspace and without any device allocation, for callers that
 * cannot allocate: code under HIP graph capture, tight serving or training loops, harnesses that
 * forbid hipMalloc. Same arguments, arithmetic and results as lcsa_attn_bwd (bit for bit), minus
 * workspace/workspace_bytes. The workspace is a static device array of LCSA_NOALLOC_SCRATCH_BYTES
 * per GPU inside the library, held from the first call on that device until the process ends; its
 * address is looked up once per device (the current device at the call). Problems whose workspace
 * (lcsa_attn_bwd_workspace_size) exceeds that size return LCSA_ERR_UNSUPPORTED before any launch.
 * Every call on one GPU shares the array: calls that overlap in time on one GPU (on different
 * streams, or from different threads) race and give wrong gradients; order them on one stream.
 * The array needs no initial contents (each call writes what it reads). */
#define LCSA_NOALLOC_SCRATCH_BYTES (16u << 20)
lcsa_status lcsa_attn_bwd_noalloc(const lcsa_problem* p, const void* q, lcsa_strides qs, const void* k,
                                  lcsa_strides ks, const void* v, lcsa_strides vs, const void* o,
                                  lcsa_strides os, const void* d_o, lcsa_strides dos, const float* lse,
                                  const int32_t* row_ptr, const int32_t* col_idx, float* dq, float* dk,
                                  float* dv, void* stream);

/* Streaming state. FlashVSR processes video as a stream of chunks; the attention of a chunk reads
 * the cached K/V of earlier chunks (fmread summary, sec. 2.2 Stage 3: temporal consistency is
 * refined through the KV cache of later layers; sec. 3, efficiency analysis: streaming adds only an
 * 8-frame lookahead, i.e. one temporal block of latent frames per chunk).
 * The cache keeps the newest `cache_tblocks` temporal blocks (2 latent frames each) of K and V and
 * the pooled K of those blocks, so each push pools only the new block's K.
 *
 * After the n-th push (w = min(n, cache_tblocks) blocks held), lcsa_stream_window describes the
 * current chunk as an ordinary problem: kv_frames = 2w (the held blocks, oldest first),
 * q_frame0 = 2(w - 1), q_frames = 2 (the newest block), and K, V, pooled K as device views into the
 * state. lcsa_pool(q only), lcsa_score_select and lcsa_attn_fwd on that window give the chunk's
 * output; they equal the same calls on K/V of the w newest blocks laid out contiguously, bit for
 * bit. Blocks older than the window are evicted (invisible to later chunks).
 *
 * Memory: the caller allocates `mem` (device, 256-byte aligned, lcsa_stream_state_size bytes) and the
 * lcsa_stream struct (host); the library keeps no other state. Inside `mem`: K and V rings of
 * `ring_tblocks` (>= 2*cache_tblocks - 1) block slots per (batch, head), filled in order; the held
 * blocks are always consecutive slots, so the window is one strided view. When the write position
 * reaches the end, the newest cache_tblocks - 1 blocks are copied to the front (a larger ring makes
 * this rarer: HBM capacity traded for bandwidth). Two pooled-K buffers are used alternately.
 * Calls on one state must be ordered on one stream.
 * chunk: batch, heads, head_dim, grid, window, topk/keep_ratio, scale, dtype of every chunk;
 *        q_frames must be 2; kv_frames and q_frame0 are ignored. */
typedef struct {
  lcsa_problem chunk;
  int32_t cache_tblocks;  /* >= 1 */
  int32_t ring_tblocks;   /* >= max(1, 2 * cache_tblocks - 1) */
  int32_t held;           /* blocks currently held, min(pushed, cache_tblocks) */
  int32_t wpos;           /* ring slot the next block goes to (ring_tblocks: compaction due) */
  int64_t pushed;         /* blocks pushed since init */
  void* mem;
  size_t mem_bytes;
} lcsa_stream;

lcsa_status lcsa_stream_state_size(const lcsa_problem* chunk, int32_t cache_tblocks, int32_t ring_tblocks,
                                   size_t* bytes);
/* Validates and resets *s (held = pushed = wpos = 0); no device work. */
lcsa_status lcsa_stream_init(lcsa_stream* s, const lcsa_problem* chunk, int32_t cache_tblocks,
                             int32_t ring_tblocks, void* mem, size_t mem_bytes);
/* Device views [B, Hh, 2*H*W, d] of the ring slot the next pushed block occupies, so that a producer
 * (e.g. the QKV projection) can write K and V there directly. Compacts the ring first when it is full
 * (asynchronous on `stream`). Any of the outputs may be NULL. */
lcsa_status lcsa_stream_reserve(lcsa_stream* s, void** k_slot, lcsa_strides* ks, void** v_slot,
                                lcsa_strides* vs, void* stream);
/* Appends one temporal block: k_new, v_new [B, Hh, 2*H*W, d] of the chunk's dtype (lcsa_strides as
 * for lcsa_attn_fwd). When they are the views lcsa_stream_reserve returned, nothing is copied;
 * otherwise they are copied into the slot. Pools k_new into the new pooled-K buffer after the kept
 * part of the old one. Asynchronous on `stream`; *s is updated on the host at once. */
lcsa_status lcsa_stream_push(lcsa_stream* s, const void* k_new, lcsa_strides ks, const void* v_new,
                             lcsa_strides vs, void* stream);
/* The current chunk as a problem and device views (valid until the next reserve or push). Fails
 * with LCSA_ERR_INVALID before the first push. */
lcsa_status lcsa_stream_window(const lcsa_stream* s, lcsa_problem* window, const void** k, lcsa_strides* ks,
                               const void** v, lcsa_strides* vs, const float** k_pooled);

/* 3D rotary position embedding and head split for a DiT attention layer feeding LCSA. The pages
 * place LCSA in the self-attention of a Wan2.1 DiT (fmread summary, sec. 2.2 Stage 1) whose queries
 * and keys carry rotary position embeddings over (time, height, width) (sec. 2.3 discusses their
 * periodicity at high resolution); the projection and RoPE precede the pooling.
 * Rotary dims: head_dim = dim_t + dim_h + dim_w (each even); the pairs (x[2i], x[2i+1]) of the
 * first dim_t/2 pairs rotate by f * theta^(-2i/dim_t), the next dim_h/2 pairs by
 * h * theta^(-2i'/dim_h), the last dim_w/2 pairs by w * theta^(-2i''/dim_w), where (f, h, w) is the
 * token's absolute latent frame and spatial position. */
typedef struct {
  int32_t dim_t, dim_h, dim_w;
  float theta;
} lcsa_rope;

/* qkv: bf16 device tensor of tokens of latent frames [frame0, frame0 + frames) of one chunk,
 * token n (raster order within those frames) of batch b at qkv + b*qkv_batch + n*qkv_token,
 * holding [3][heads][head_dim] (q, k, v), the layout a [tokens, 3*heads*head_dim] projection
 * output has. Writes rope(q), rope(k) and v as [B, heads, frames*H*W, head_dim] bf16 with the given
 * strides (for example into lcsa_stream_reserve's slot). Computes in fp32, rounds once to bf16.
 * p supplies batch, heads, head_dim, grid and dtype (bf16 only); frames is even (>= 2). */
lcsa_status lcsa_rope_qkv(const lcsa_problem* p, const lcsa_rope* rope, const void* qkv, int64_t qkv_batch,
                          int64_t qkv_token, int32_t frame0, int32_t frames, void* q, lcsa_strides qs,
                          void* k, lcsa_strides ks, void* v, lcsa_strides vs, void* stream);

const char* lcsa_status_string(lcsa_status s);
const char* lcsa_last_error(void);   /* thread-local detail of this thread's last non-OK return */
int32_t lcsa_version(void);          /* major*10000 + minor*100 + patch */

#ifdef __cplusplus
}
#endif
#endif /* LCSA_H_ */
