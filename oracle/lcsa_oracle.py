"""CPU fp64 oracle for the LCSA forward pass (locality-constrained block-sparse causal attention).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module. The product path (the HIP library and its Python binding) never calls it, and
it shares no code with that path: the two meet only on the seeded input arrays.

Source: "FlashVSR: Towards Real-time Diffusion-Based Streaming Video Super Resolution", the
fmread pdfshare summary of the paper:
  * sec. 2.2, Stage 2, causal masking: every latent attends only to the current and earlier times.
  * sec. 2.2, Stage 2, block-sparse attention: Q and K are cut into non-overlapping blocks
    (2x8x8 in the example), average-pooled to one feature per block, a coarse block-to-block
    attention map is formed, the Top-K most relevant block pairs are kept and full attention runs
    inside the kept blocks only.
  * sec. 2.3, locality-constrained attention: at inference each query's attention is confined to a
    local spatial neighbourhood (1152x1152 px in the example), with a "boundary-truncated" and a
    "boundary-preserving" rule compared in sec. 3 (ablation, locality-constrained attention).
The passages leave several steps open; the readings taken here are:
  R1 causality is block-causal: key block j is visible from query block i iff its temporal block
     index (latent frame // 2) is <= that of i; a block is fully visible inside the current one.
  R2 Top-K is taken per query block over its visible key blocks, independently per (batch, head).
  R3 K_i = min(topk, n_i) when a fixed topk is given, else clamp(floor(rho*n_i + 0.5), 1, n_i), with
     n_i the number of visible key blocks; rho is the keep ratio (13.6% in the ablation).
  R4 the coarse block map is the scaled dot product of the pooled vectors; a row softmax of it is
     monotone and would not change the Top-K, so selection works on the logits.
  R5 exact score ties go to the lower key-block index; no block is forced in.
  R6 the window is block-granular and spatial only, w_b = win/8 blocks (odd), r = (w_b - 1)/2,
     applied to the block rows and columns independently and identically in every visible
     temporal block. Truncated: blocks within r of the query block, cut at the frame edge.
     Preserving: a w_b-wide window slid inward at the edge, start = clamp(c - r, 0, N - w_b),
     so every query keeps w_b blocks per axis when the grid has that many.
  R7 the pooled feature is the arithmetic mean of the block's 128 tokens.
  R10 (the attention layer around LCSA) Q and K carry a rotary position embedding over (time,
     height, width): the head dim splits into three even groups, one per axis; adjacent dims form
     the rotated pairs; frequencies theta^(-2j/dim_axis); positions are the absolute latent frame
     and the token row and column. The pages only name the embedding (sec. 2.3).
  R11 token-granular windows (the same two rules per token): a query token at position c of an axis
     of n tokens sees the w tokens starting at c - (w-1)//2, cut to [0, n) (truncated) or shifted
     inside (preserving); a key block is a candidate of a query block when some token of one sees
     some token of the other (block-causal as before); inside kept blocks only visible token pairs
     take part; a query token that sees no kept token gets O = 0 and lse = -inf.
  R9 a grid that is not a multiple of 8 is cut into blocks from its origin; the last block row and
     column are partial. A partial block is pooled over the tokens it has, and attention over a
     kept partial block covers only those tokens. Block counts are ceil(H/8) x ceil(W/8).
Every function works in fp64 on exact copies of the kernel inputs.

The backward (`attend_bwd`) is not described by the sources: it is the exact gradient of `attend`
for a fixed selection, written out from the definition of softmax attention (the selection
itself is discrete and not differentiated).

Streaming (`stream_forward`): the summary's sec. 2.2 Stage 3 refines temporal consistency through the
KV cache, and sec. 3 (efficiency analysis) streams with an 8-frame lookahead. Reading R8: each chunk
adds one temporal block (2 latent frames); the chunk's queries are that block and its keys/values
are the cached blocks plus the new one, at most `cache_tblocks` blocks, older ones evicted. The chunk
output is then the forward above on that window, with frames counted from the window's first frame.
"""
from __future__ import annotations

import numpy as np

BLK_T, BLK_H, BLK_W = 2, 8, 8
BLK = BLK_T * BLK_H * BLK_W
WIN_NONE, WIN_TRUNCATED, WIN_PRESERVING = 0, 1, 2
WIN_TOKEN_TRUNCATED, WIN_TOKEN_PRESERVING = 3, 4


# ----------------------------------------------------------------------------------- geometry
def _grid(p):
    """Blocks per frame along h and w: the grid is cut from its origin, the last block row/column
    may be partial (R9)."""
    hb, wb = -(-p.grid_h // BLK_H), -(-p.grid_w // BLK_W)
    return hb, wb


def query_blocks(p):
    """(tb, hb, wb) of every query block, in block-index order i = (tb_rel*Hb + hb)*Wb + wb.

    tb is the ABSOLUTE temporal block (latent frame // 2); Q starts at latent frame q_frame0.
    """
    Hb, Wb = _grid(p)
    out = []
    for tr in range(p.q_frames // BLK_T):
        for hb in range(Hb):
            for wb in range(Wb):
                out.append((p.q_frame0 // BLK_T + tr, hb, wb))
    return out


def key_blocks(p):
    """(tb, hb, wb) of every key block, j = (tb*Hb + hb)*Wb + wb; K/V start at latent frame 0."""
    Hb, Wb = _grid(p)
    return [(tb, hb, wb) for tb in range(p.kv_frames // BLK_T) for hb in range(Hb) for wb in range(Wb)]


def window_blocks(mode, c, n, wb_size):
    """Set of block coordinates along one axis (of n blocks) that a query at block c may see (R6)."""
    if mode == WIN_NONE:
        return set(range(n))
    r = (wb_size - 1) // 2
    if mode == WIN_TRUNCATED:
        return {x for x in range(n) if abs(x - c) <= r}
    if mode == WIN_PRESERVING:
        if n <= wb_size:
            return set(range(n))
        start = min(max(c - r, 0), n - wb_size)
        return set(range(start, start + wb_size))
    raise ValueError(mode)


def token_window(mode, c, n, w):
    """Set of token coordinates along one axis (of n tokens) that a query token at c sees (R11)."""
    start = c - (w - 1) // 2
    if mode == WIN_TOKEN_TRUNCATED:
        return {x for x in range(start, start + w) if 0 <= x < n}
    if mode == WIN_TOKEN_PRESERVING:
        if n <= w:
            return set(range(n))
        start = min(max(start, 0), n - w)
        return set(range(start, start + w))
    raise ValueError(mode)


def _token_axis_blocks(p, mode, c_block, n_tok, w):
    """Block coordinates along one axis seen by some token of block c_block (R11)."""
    seen = set()
    for c in range(c_block * BLK_H, min(c_block * BLK_H + BLK_H, n_tok)):
        seen |= token_window(mode, c, n_tok, w)
    return {x // BLK_H for x in seen}


def visible(p):
    """Boolean [nqb, nkb]: block-causal (R1) AND spatial window (R6 / R11), by enumeration."""
    Hb, Wb = _grid(p)
    qb, kb = query_blocks(p), key_blocks(p)
    if p.win_mode >= WIN_TOKEN_TRUNCATED:
        vis = np.zeros((len(qb), len(kb)), dtype=bool)
        for i, (ti, hi, wi) in enumerate(qb):
            rows = _token_axis_blocks(p, p.win_mode, hi, p.grid_h, p.win_h)
            cols = _token_axis_blocks(p, p.win_mode, wi, p.grid_w, p.win_w)
            for j, (tj, hj, wj) in enumerate(kb):
                vis[i, j] = (tj <= ti) and (hj in rows) and (wj in cols)
        return vis
    wh = p.win_h // BLK_H if p.win_mode != WIN_NONE else 0
    ww = p.win_w // BLK_W if p.win_mode != WIN_NONE else 0
    vis = np.zeros((len(qb), len(kb)), dtype=bool)
    for i, (ti, hi, wi) in enumerate(qb):
        rows = window_blocks(p.win_mode, hi, Hb, wh)
        cols = window_blocks(p.win_mode, wi, Wb, ww)
        for j, (tj, hj, wj) in enumerate(kb):
            vis[i, j] = (tj <= ti) and (hj in rows) and (wj in cols)
    return vis


def keep_count(p, n: int) -> int:
    """K_i for a row with n visible key blocks (R3); the ratio rule is evaluated in fp64."""
    if p.topk > 0:
        return min(p.topk, n)
    x = float(p.keep_ratio) * float(n)
    x = x + 0.5
    return int(min(max(np.floor(x), 1), n))


def csr_row_ptr(p, vis=None):
    """row_ptr[nqb+1]: exclusive prefix sum of K_i (the same for every batch and head)."""
    vis = visible(p) if vis is None else vis
    k = [keep_count(p, int(n)) for n in vis.sum(axis=1)]
    return np.concatenate([[0], np.cumsum(k)]).astype(np.int64)


def block_tokens(p, blk, frame0):
    """Token indices (raster order n = (t*H + h)*W + w) of block (tb, hb, wb) in a tensor whose
    first latent frame is `frame0`; only the tokens inside the H x W grid (R9)."""
    tb, hb, wb = blk
    H, W = p.grid_h, p.grid_w
    idx = []
    for t in range(tb * BLK_T, tb * BLK_T + BLK_T):
        for h in range(hb * BLK_H, min(hb * BLK_H + BLK_H, H)):
            for w in range(wb * BLK_W, min(wb * BLK_W + BLK_W, W)):
                idx.append(((t - frame0) * H + h) * W + w)
    return np.array(idx, dtype=np.int64)


# ---------------------------------------------------------------------------------- pooling
def pool(p, x, which: str):
    """Mean of each block's tokens (R7: 128, fewer in a partial edge block, R9). x: [B, heads, N, d] -> [B, heads, nblk, d] fp64."""
    x = np.asarray(x, dtype=np.float64)
    blocks, f0 = (query_blocks(p), p.q_frame0) if which == "q" else (key_blocks(p), 0)
    out = np.empty(x.shape[:2] + (len(blocks), x.shape[3]), dtype=np.float64)
    for n, blk in enumerate(blocks):
        out[:, :, n, :] = x[:, :, block_tokens(p, blk, f0), :].mean(axis=2)
    return out


# ------------------------------------------------------------------------- score + select
def block_scores(p, qbar, kbar, vis=None):
    """Coarse block map s_ij = scale * <qbar_i, kbar_j> (R4); -inf where j is not visible."""
    vis = visible(p) if vis is None else vis
    s = p.scale * np.matmul(qbar, np.swapaxes(kbar, -1, -2))
    return np.where(vis[None, None], s, -np.inf)


def select(p, scores, vis=None):
    """Per (batch, head, query block): the K_i visible key blocks first in the order
    (score descending, index ascending) (R2, R5); returned ascending in j, concatenated per row.

    Returns (row_ptr [nqb+1], col_idx [B, heads, nnz]).
    """
    vis = visible(p) if vis is None else vis
    row_ptr = csr_row_ptr(p, vis)
    B, Hh, nqb, _ = scores.shape
    col = np.empty((B, Hh, int(row_ptr[-1])), dtype=np.int64)
    for b in range(B):
        for h in range(Hh):
            for i in range(nqb):
                cand = np.flatnonzero(vis[i])
                k = int(row_ptr[i + 1] - row_ptr[i])
                order = np.lexsort((cand, -scores[b, h, i, cand]))  # primary: -score, then j
                col[b, h, row_ptr[i]:row_ptr[i + 1]] = np.sort(cand[order[:k]])
    return row_ptr, col


# -------------------------------------------------------------------------------- attention
def token_pair_mask(p, qt, kt):
    """[len(qt), len(kt)] boolean: query token qt[a] sees key token kt[b] under a token-granular
    window (R11); all True for the block-granular modes. Token indices are raster positions in their
    own tensors, so only the spatial coordinates matter here (causality is block-level)."""
    if p.win_mode < WIN_TOKEN_TRUNCATED:
        return np.ones((len(qt), len(kt)), dtype=bool)
    hw = p.grid_h * p.grid_w
    hq, wq = (qt % hw) // p.grid_w, qt % p.grid_w
    hk, wk = (kt % hw) // p.grid_w, kt % p.grid_w
    # each window is a run of consecutive coordinates: keep its first and last
    rows = [token_window(p.win_mode, h, p.grid_h, p.win_h) for h in range(p.grid_h)]
    cols = [token_window(p.win_mode, w, p.grid_w, p.win_w) for w in range(p.grid_w)]
    rlo, rhi = np.array([min(r) for r in rows]), np.array([max(r) for r in rows])
    clo, chi = np.array([min(c) for c in cols]), np.array([max(c) for c in cols])
    mh = (hk[None, :] >= rlo[hq][:, None]) & (hk[None, :] <= rhi[hq][:, None])
    mw = (wk[None, :] >= clo[wq][:, None]) & (wk[None, :] <= chi[wq][:, None])
    return mh & mw


def attend(p, q, k, v, row_ptr, col_idx, qblocks=None, bh=None):
    """Exact softmax attention of every query token of block i over all tokens of the key blocks
    listed for row i (no token-level mask inside a selected block, except the token-granular window
    of R11).

    q: [B, heads, Nq, d], k/v: [B, heads, Nk, d]. Returns O [B, heads, Nq, d] and lse [B, heads, Nq]
    (natural log of the softmax denominator, max-shifted); rows not requested stay NaN.
    qblocks: iterable of query-block indices to compute (default: all).
    bh: iterable of (batch, head) pairs to compute (default: all).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hh, Nq, d = q.shape
    qb, kb = query_blocks(p), key_blocks(p)
    O = np.full(q.shape, np.nan)
    lse = np.full(q.shape[:3], np.nan)
    qblocks = range(len(qb)) if qblocks is None else qblocks
    bh = [(b, h) for b in range(B) for h in range(Hh)] if bh is None else bh
    ktok = [block_tokens(p, blk, 0) for blk in kb]
    for i in qblocks:
        qt = block_tokens(p, qb[i], p.q_frame0)
        for b, h in bh:
            sel = col_idx[b, h, row_ptr[i]:row_ptr[i + 1]]
            kt = np.concatenate([ktok[j] for j in sel])
            logits = p.scale * (q[b, h, qt] @ k[b, h, kt].T)      # [128, K_i*128]
            mask = token_pair_mask(p, qt, kt)
            logits = np.where(mask, logits, -np.inf)
            m = logits.max(axis=1, keepdims=True)
            seen = np.isfinite(m)                                  # rows that see some kept token
            e = np.exp(logits - np.where(seen, m, 0.0))
            den = e.sum(axis=1, keepdims=True)
            O[b, h, qt] = np.where(seen, (e / np.where(seen, den, 1.0)) @ v[b, h, kt], 0.0)
            lse[b, h, qt] = np.where(seen, m + np.log(np.where(seen, den, 1.0)), -np.inf)[:, 0]
    return O, lse


def attend_bwd(p, q, k, v, row_ptr, col_idx, dO, qblocks=None, bh=None):
    """Gradients of `attend` for a fixed selection: given dL/dO, returns dL/dQ, dL/dK, dL/dV (fp64).

    The selection (row_ptr, col_idx) is an input, not differentiated. For each query token t of block
    i and the tokens k of its kept blocks, with logits s = scale*q.k, P = softmax(s) and O = P V:
      dV_k += sum_t P_tk dO_t,  dP_tk = dO_t . v_k,  Delta_t = dO_t . O_t = sum_k P_tk dP_tk,
      dS_tk = P_tk (dP_tk - Delta_t),  dQ_t = scale sum_k dS_tk k_k,  dK_k += scale sum_t dS_tk q_t.
    dK and dV sum over every query block that kept the key block. With `qblocks` only those query
    blocks contribute (dQ of the other rows stays NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    qb, kb = query_blocks(p), key_blocks(p)
    dQ = np.full(q.shape, np.nan)
    dK = np.zeros(k.shape)
    dV = np.zeros(v.shape)
    qblocks = range(len(qb)) if qblocks is None else qblocks
    B, Hh = q.shape[:2]
    bh = [(b, h) for b in range(B) for h in range(Hh)] if bh is None else bh
    ktok = [block_tokens(p, blk, 0) for blk in kb]
    for i in qblocks:
        qt = block_tokens(p, qb[i], p.q_frame0)
        for b, h in bh:
            sel = col_idx[b, h, row_ptr[i]:row_ptr[i + 1]]
            kt = np.concatenate([ktok[j] for j in sel])
            logits = p.scale * (q[b, h, qt] @ k[b, h, kt].T)
            logits = np.where(token_pair_mask(p, qt, kt), logits, -np.inf)
            m = logits.max(axis=1, keepdims=True)
            seen = np.isfinite(m)                                   # rows that see some kept token
            e = np.exp(logits - np.where(seen, m, 0.0))
            P = e / np.where(seen, e.sum(axis=1, keepdims=True), 1.0)  # [128, n]; unseen rows are 0
            Ot = P @ v[b, h, kt]
            g = dO[b, h, qt]
            dP = g @ v[b, h, kt].T
            delta = (g * Ot).sum(axis=1, keepdims=True)
            dS = P * (dP - delta)
            dQ[b, h, qt] = p.scale * (dS @ k[b, h, kt])
            dK[b, h, kt] += p.scale * (dS.T @ q[b, h, qt])
            dV[b, h, kt] += P.T @ g
    return dQ, dK, dV


def forward(p, q, k, v, qblocks=None, bh=None):
    """The whole path: pool -> score -> mask -> Top-K -> exact attention on the kept blocks."""
    vis = visible(p)
    qbar, kbar = pool(p, q, "q"), pool(p, k, "k")
    s = block_scores(p, qbar, kbar, vis)
    row_ptr, col = select(p, s, vis)
    O, lse = attend(p, q, k, v, row_ptr, col, qblocks=qblocks, bh=bh)
    return dict(vis=vis, qbar=qbar, kbar=kbar, scores=s, row_ptr=row_ptr, col_idx=col, O=O, lse=lse)


def stream_window(p, c: int, cache_tblocks: int):
    """(first temporal block, problem) of streaming chunk c (0-based): the window holds temporal blocks
    first..c, first = max(0, c - cache_tblocks + 1); the queries are block c (R8)."""
    import copy
    import dataclasses
    first = max(0, c - cache_tblocks + 1)
    w = c - first + 1
    frames = dict(kv_frames=BLK_T * w, q_frame0=BLK_T * (w - 1), q_frames=BLK_T)
    if dataclasses.is_dataclass(p):
        return first, dataclasses.replace(p, **frames)
    pw = copy.copy(p)
    for name, val in frames.items():
        setattr(pw, name, val)
    return first, pw


def stream_forward(p, q_seq, k_seq, v_seq, cache_tblocks: int, chunks=None):
    """Chunk-by-chunk LCSA over a sequence (R8). q_seq, k_seq, v_seq: [B, heads, T*H*W, d], latent
    frames 0..T-1 in raster order. Chunk c's queries are frames 2c, 2c+1; its keys and values are the
    frames of `stream_window`. Returns {c: forward(...) of that window}."""
    hw = p.grid_h * p.grid_w
    tbt = BLK_T * hw
    T = q_seq.shape[2] // hw
    chunks = range(T // BLK_T) if chunks is None else chunks
    out = {}
    for c in chunks:
        first, pw = stream_window(p, c, cache_tblocks)
        q = q_seq[:, :, c * tbt:(c + 1) * tbt]
        k = k_seq[:, :, first * tbt:(c + 1) * tbt]
        v = v_seq[:, :, first * tbt:(c + 1) * tbt]
        out[c] = forward(pw, q, k, v)
    return out


def rope_3d(p, x, frame0: int, dims, theta: float):
    """3D rotary position embedding (R10) of x [B, heads, N, d] whose tokens are latent frames
    frame0, frame0 + 1, ... of a grid_h x grid_w grid in raster order. dims = (dim_t, dim_h, dim_w),
    summing to d: pair i = (x[2i], x[2i+1]) of the first dim_t/2 pairs turns by f * theta^(-2i/dim_t)
    (f the absolute frame), the next dim_h/2 pairs by h * theta^(-2i'/dim_h), the last dim_w/2 by
    w * theta^(-2i''/dim_w); a turn by a maps (x0, x1) to (x0 cos a - x1 sin a, x0 sin a + x1 cos a)."""
    x = np.asarray(x, dtype=np.float64)
    H, W = p.grid_h, p.grid_w
    n = np.arange(x.shape[2])
    pos = {"t": frame0 + n // (H * W), "h": (n % (H * W)) // W, "w": n % W}
    angles = []
    for axis, dim in zip("thw", dims):
        for j in range(dim // 2):
            angles.append(pos[axis] * float(theta) ** (-2.0 * j / dim))
    ang = np.stack(angles, axis=1)                    # [N, d/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def dense_block_causal(p, q, k, v):
    """Dense attention with the token mask induced by block visibility (every key token of a
    visible block, no selection). With keep ratio 1 LCSA must reduce to this. Small inputs only."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    vis = visible(p)
    Nq, Nk = q.shape[2], k.shape[2]
    qblock_of = np.empty(Nq, dtype=np.int64)
    kblock_of = np.empty(Nk, dtype=np.int64)
    for i, blk in enumerate(query_blocks(p)):
        qblock_of[block_tokens(p, blk, p.q_frame0)] = i
    for j, blk in enumerate(key_blocks(p)):
        kblock_of[block_tokens(p, blk, 0)] = j
    mask = vis[qblock_of][:, kblock_of]                                # [Nq, Nk]
    mask &= token_pair_mask(p, np.arange(Nq), np.arange(Nk))          # token-granular window (R11)
    logits = p.scale * np.matmul(q, np.swapaxes(k, -1, -2))
    logits = np.where(mask, logits, -np.inf)
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    den = e.sum(axis=-1, keepdims=True)
    return np.matmul(e / den, v), (m + np.log(den))[..., 0]
