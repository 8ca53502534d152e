"""GPU parity: the HIP path through the C ABI against the fp64 oracle (tolerances in tests/parity.py).

Workloads at full size run the same launch configuration the benchmark times; attention is compared
on sampled query blocks there (every head), and on every row for the smaller cases.
"""
import json
import sys

import numpy as np
import pytest
import torch

from block_sparse_causal_lcsa_amd import inputs, lcsa
from block_sparse_causal_lcsa_amd import workloads as W
from oracle import lcsa_oracle as O

from parity import check_attention, check_pooled, check_selection, full_check, run_gpu, to_device, from_device

pytestmark = pytest.mark.gpu


def report(name, stats):
    print(f"PARITY {name} {json.dumps(stats)}", flush=True)
    sys.stdout.flush()


def sample_blocks(w, n=10, seed=0):
    """First, last, one per temporal block edge and random interior query blocks."""
    rng = np.random.default_rng(seed)
    nqb, bpt = w.nqb, w.blocks_per_tblock
    pick = {0, nqb - 1, bpt - 1, nqb - bpt}
    pick |= set(rng.choice(nqb, size=min(n, nqb), replace=False).tolist())
    return sorted(pick)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tiny(seed):
    report(f"{W.TINY.name}/seed{seed}", full_check(W.TINY, seed))


@pytest.mark.parametrize("seed", [0, 1])
def test_chunk_768x1408(seed):
    w = W.CHUNK_768
    qb = None if seed == 0 else sample_blocks(w, seed=seed)
    report(f"{w.name}/seed{seed}", full_check(w, seed, qblocks=qb))


@pytest.mark.parametrize("w", [W.UHD_TRUNC, W.UHD_PRES], ids=lambda w: w.name)
def test_uhd_window(w):
    # corner, edge and interior blocks of both query frames
    Wb = w.grid_w // 8
    qb = sorted({0, Wb - 1, 3 * Wb + 5, 5 * Wb + 10, 11 * Wb + 20, 6 * Wb, 11 * Wb, w.nqb - 1}
                | set(sample_blocks(w, 4)))
    report(w.name, full_check(w, 0, qblocks=qb))


@pytest.mark.parametrize("rho", W.SWEEP_RHOS)
def test_sweep_768x1408_8f(rho):
    w = W.sweep(rho)
    stats = full_check(w, 0, qblocks=sample_blocks(w, 6), bh=[(0, h) for h in (0, 5, 11)])
    report(w.name, stats)


def test_clip_768x1408_26f():
    w = W.CLIP_768
    qb = sample_blocks(w, 8) + [66 * 6 + 30, 66 * 12 + 65]
    stats = full_check(w, 0, qblocks=sorted(set(qb)), bh=[(0, h) for h in (0, 7)], scores=False)
    report(w.name, stats)


# Beyond the former 1,248-key-block row limit: a 12-frame K/V cache at 1536x2688 with the 72-token
# truncated window (1,512 key blocks, at most 6 x 81 candidates per query block), and a 40-frame cache
# at 768x1408 without a window (1,320 key blocks, all of them candidates).
LONG = [
    W.Workload("uhd_1536x2688_kv12_win72_truncated", 1, 12, 128, 96, 168, 12, 10, 2, win_mode=1, win_h=72,
               win_w=72, keep_ratio=W.RHO),
    W.Workload("chunk_768x1408_kv40", 1, 12, 128, 48, 88, 40, 38, 2, keep_ratio=W.RHO),
]


@pytest.mark.parametrize("w", LONG, ids=lambda w: w.name)
def test_long_caches(w):
    assert w.nkb > 1248
    stats = full_check(w, 0, qblocks=sample_blocks(w, 8), bh=[(0, h) for h in (0, 6, 11)])
    report(w.name, stats)


# Rows with more candidates than the selection's register slots hold (over 2,048: it rereads the row's
# scores from LDS on every pass), and a tile whose four-row union would overflow LDS (over 5,118
# candidates: single-row tiles). Pool and selection against the oracle; attention is unaffected by
# the row length and covered above.
BEYOND = [
    W.Workload("chunk_768x1408_kv66_rows_in_lds", 1, 1, 128, 48, 88, 66, 64, 2, keep_ratio=W.RHO),
    W.Workload("grid_8x8_kv10242_single_row_tiles", 1, 1, 64, 8, 8, 10242, 10240, 2, keep_ratio=0.01),
]


@pytest.mark.parametrize("w", BEYOND, ids=lambda w: w.name)
def test_selection_beyond_register_slots(w):
    x = inputs.make_inputs(w, 0, want=("q", "k"))
    p = lcsa.problem(w)
    nqb, nkb, nnz, rp = lcsa.lcsa_csr_layout(p)
    assert int(np.max(np.diff(rp))) >= 1 and nkb > 2048
    q, k = to_device(x["q"]), to_device(x["k"])
    qp, kp = lcsa.lcsa_pool(p, q, k)
    col = lcsa.lcsa_score_select(p, qp, kp, torch.from_numpy(rp).to("cuda"))
    torch.cuda.synchronize()
    gpu = dict(row_ptr=rp.astype(np.int64), col_idx=col.cpu().numpy().astype(np.int64))
    vis = O.visible(w)
    assert int(vis.sum(axis=1).max()) > 2048
    qbar, kbar = O.pool(w, inputs.to_f64(x["q"]), "q"), O.pool(w, inputs.to_f64(x["k"]), "k")
    check_pooled(w, qp.cpu().numpy(), qbar)
    check_pooled(w, kp.cpu().numpy(), kbar)
    s = O.block_scores(w, qbar, kbar, vis)
    rp_o, col_o = O.select(w, s, vis)
    near, swapped = check_selection(w, gpu, s, col_o, rp_o)
    report(w.name, dict(near_tie_rows=near, swapped_rows=swapped))


def test_full_selection_is_dense_block_causal():
    """keep ratio 1 on the GPU equals the oracle's dense masked attention (no selection)."""
    w = W.Workload("dense_small", 1, 2, 128, 24, 32, 6, 0, 6, keep_ratio=1.0)
    x = inputs.make_inputs(w, 3)
    gpu = run_gpu(w, x)
    Od, lsed = O.dense_block_causal(w, *(inputs.to_f64(x[n]) for n in "qkv"))
    dO = np.abs(gpu["O"] - Od)
    assert dO.max() <= 2e-2 and dO.mean() <= 2e-3
    assert np.abs(gpu["lse"] - lsed).max() <= 1e-3


# ------------------------------------------------------------------------------- edge cases
EDGE = [
    # ragged query tiles (nqb not a multiple of 16) and key slots (nkb not a multiple of 64)
    W.Workload("ragged_40x56_q2of6", 1, 2, 128, 40, 56, 6, 4, 2, keep_ratio=0.3),
    # queries in the middle of the key frames (later key frames are never visible)
    W.Workload("mid_q2_kv8", 1, 2, 128, 16, 24, 8, 2, 2, keep_ratio=0.5),
    # windows smaller and larger than the grid, both rules
    W.Workload("win_trunc_small", 1, 2, 128, 56, 40, 4, 2, 2, win_mode=1, win_h=24, win_w=40, keep_ratio=0.4),
    W.Workload("win_pres_small", 1, 2, 128, 56, 40, 4, 2, 2, win_mode=2, win_h=24, win_w=40, keep_ratio=0.4),
    W.Workload("win_wider_than_grid", 1, 1, 128, 16, 24, 4, 0, 4, win_mode=2, win_h=72, win_w=72, keep_ratio=0.5),
    # fixed Top-K: K = 1 and K larger than every n_i
    W.Workload("topk1", 1, 2, 128, 16, 32, 4, 0, 4, topk=1),
    W.Workload("topk_all", 1, 2, 128, 16, 32, 4, 0, 4, topk=50),
    # other head size / dtype combinations, batch > 1
    W.Workload("d64_bf16_b2", 2, 3, 64, 16, 24, 4, 0, 4, keep_ratio=0.5),
    W.Workload("d128_f32", 1, 2, 128, 16, 24, 4, 2, 2, dtype="f32", keep_ratio=0.5),
    # the largest key count a selection row holds (1188 key blocks, 18 temporal blocks)
    W.Workload("max_keys_768x1408_kv36", 1, 1, 128, 48, 88, 36, 34, 2, keep_ratio=0.05),
    # an odd number of (batch, head, query block) rows: the last workgroup's second query block is
    # empty; with a truncated window the two rows of a workgroup keep different block counts
    W.Workload("odd_rows_24x40", 1, 1, 128, 24, 40, 4, 2, 2, keep_ratio=0.4),
    W.Workload("odd_rows_24x40_win_trunc", 1, 1, 128, 24, 40, 4, 2, 2, win_mode=1, win_h=24, win_w=24, keep_ratio=0.5),
    W.Workload("odd_rows_24x40_d64", 1, 3, 64, 24, 40, 2, 0, 2, keep_ratio=0.4),
]


@pytest.mark.parametrize("w", EDGE, ids=lambda w: w.name)
def test_edge_cases(w):
    qb = None if w.nqb <= 64 else sample_blocks(w, 8)
    report(w.name, full_check(w, 0, qblocks=qb))


# Grids that are not multiples of 8: the last block row / column is partial (its tokens inside the
# grid are pooled, attended to, and the only ones with outputs).
RAGGED = [
    W.Workload("ragged_21x37", 1, 2, 128, 21, 37, 4, 2, 2, keep_ratio=0.4),
    W.Workload("ragged_13x10_d64_win_pres", 1, 2, 64, 13, 10, 4, 0, 4, win_mode=2, win_h=24, win_w=24,
               keep_ratio=0.5),
    W.Workload("ragged_19x27_win_trunc_b2", 2, 2, 128, 19, 27, 6, 2, 4, win_mode=1, win_h=24, win_w=24,
               keep_ratio=0.4),
    W.Workload("ragged_9x7_f32", 1, 2, 128, 9, 7, 4, 2, 2, dtype="f32", keep_ratio=0.5),
    W.Workload("ragged_3x5_below_one_block", 1, 1, 128, 3, 5, 6, 4, 2, topk=2),
]


@pytest.mark.parametrize("w", RAGGED, ids=lambda w: w.name)
def test_ragged_grids(w):
    report(w.name, full_check(w, 0))


# Token-granular windows (per-token masks inside kept blocks, R11), both rules, even and odd sizes,
# with a ragged grid, d = 64 and fp32 I/O
TOKEN_WINDOWS = [
    W.Workload("tokwin_trunc_24x40_w13x17", 1, 2, 128, 24, 40, 4, 2, 2, win_mode=3, win_h=13, win_w=17,
               keep_ratio=0.5),
    W.Workload("tokwin_pres_21x37_w20x9", 1, 2, 128, 21, 37, 6, 4, 2, win_mode=4, win_h=20, win_w=9,
               keep_ratio=0.4),
    W.Workload("tokwin_trunc_16x24_w6_d64_b2", 2, 2, 64, 16, 24, 4, 0, 4, win_mode=3, win_h=6, win_w=6, topk=2),
    W.Workload("tokwin_pres_16x24_f32", 1, 2, 128, 16, 24, 4, 2, 2, dtype="f32", win_mode=4, win_h=11, win_w=24,
               keep_ratio=0.5),
]


@pytest.mark.parametrize("w", TOKEN_WINDOWS, ids=lambda w: w.name)
def test_token_windows(w):
    report(w.name, full_check(w, 0))


def test_token_window_rows_without_keys():
    """One kept block per row under a 3x3-token window: query tokens deep inside their block see none
    of a neighbouring kept block, and must get O = 0 and lse = -inf."""
    w = W.Workload("tokwin_blind_24x32_w3_topk1", 1, 2, 128, 24, 32, 4, 2, 2, win_mode=3, win_h=3, win_w=3,
                   topk=1)
    x = inputs.make_inputs(w, 0)
    x["k"] = x["k"] ^ np.uint16(0x8000)   # K negated (bf16 sign bit): a query block's own block scores lowest
    gpu = run_gpu(w, x)
    x64 = [inputs.to_f64(x[n]) for n in "qkv"]
    vis = O.visible(w)
    s = O.block_scores(w, O.pool(w, x64[0], "q"), O.pool(w, x64[1], "k"), vis)
    rp, col = O.select(w, s, vis)
    near, swapped = check_selection(w, gpu, s, col, rp)
    stats = check_attention(w, x64, gpu)
    assert stats["blind_rows"] > 0
    stats.update(near_tie_rows=near, swapped_rows=swapped)
    report(w.name, stats)


def test_uhd_token_window_72():
    """The 1536x2688 chunk with a 72x72-token window per query token (truncated), sampled rows."""
    w = W.UHD_TRUNC.replace(name="chunk_1536x2688_tokwin72_truncated", win_mode=3, win_h=72, win_w=72)
    Wb = w.grid_w // 8
    qb = sorted({0, Wb - 1, 5 * Wb + 10, 11 * Wb + 20, w.nqb - 1} | set(sample_blocks(w, 4)))
    report(w.name, full_check(w, 0, qblocks=qb, bh=[(0, h) for h in (0, 7)], scores=False))


def test_hd_720x1280_ragged():
    """A 720x1280 chunk: 45x80 latent tokens, the last block row 5 tokens deep; sampled query blocks
    include the whole last block row."""
    w = W.HD_720
    Wb = w.grid_w // 8
    last_row = [w.nqb - Wb + x for x in range(0, Wb, 3)] + [w.nqb - 1]
    qb = sorted(set(sample_blocks(w, 6)) | set(last_row))
    report(w.name, full_check(w, 0, qblocks=qb, bh=[(0, h) for h in (0, 6, 11)]))


def test_exact_ties_go_to_lower_index():
    """Constant K makes every score of a row equal: the K_i lowest visible indices must be kept."""
    w = W.Workload("ties", 1, 2, 128, 24, 32, 6, 2, 4, keep_ratio=0.25)
    x = inputs.make_inputs(w, 0)
    x["k"] = np.full_like(x["k"], x["k"].flat[0])
    gpu = run_gpu(w, x)
    vis = O.visible(w)
    rp = gpu["row_ptr"]
    for h in range(2):
        for i in range(w.nqb):
            assert list(gpu["col_idx"][0, h, rp[i]:rp[i + 1]]) == list(np.flatnonzero(vis[i])[:rp[i + 1] - rp[i]])


def test_strided_tensors():
    """Q/K/V/O as [B, tokens, heads, d] storage viewed as [B, heads, tokens, d] (token stride heads*d)."""
    w = W.Workload("strided", 2, 3, 128, 16, 24, 4, 2, 2, keep_ratio=0.5)
    x = inputs.make_inputs(w, 5)
    p = lcsa.problem(w)

    def strided(a):
        t = to_device(a).permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        assert not t.is_contiguous()
        return t

    q, k, v = (strided(x[n]) for n in "qkv")
    o = torch.empty((2, w.nq_tokens, 3, 128), dtype=torch.bfloat16, device="cuda").permute(0, 2, 1, 3)
    ref = run_gpu(w, x)
    rp = torch.from_numpy(lcsa.lcsa_csr_layout(p)[3]).cuda()
    qp, kp = lcsa.lcsa_pool(p, q, k)
    col = lcsa.lcsa_score_select(p, qp, kp, rp)
    _, lse = lcsa.lcsa_attn_fwd(p, q, k, v, rp, col, o=o)
    torch.cuda.synchronize()
    assert np.array_equal(qp.cpu().numpy(), ref["qbar"]) and np.array_equal(kp.cpu().numpy(), ref["kbar"])
    assert np.array_equal(col.cpu().numpy(), ref["col_idx"])
    assert np.array_equal(from_device(o), ref["O"])
    assert np.array_equal(lse.cpu().numpy(), ref["lse"])


def test_deterministic_and_causal():
    """Two runs are bit-identical; changing Q/K/V of the last temporal block leaves every earlier
    query row, its selection and its lse bit-identical."""
    w = W.Workload("causal", 1, 2, 128, 24, 40, 6, 0, 6, keep_ratio=0.3)
    x = inputs.make_inputs(w, 1)
    a, b = run_gpu(w, x), run_gpu(w, x)
    for key in ("qbar", "kbar", "col_idx", "O", "lse"):
        assert np.array_equal(a[key], b[key]), key
    hw = w.grid_h * w.grid_w
    y = {n: x[n].copy() for n in "qkv"}
    rng = np.random.default_rng(0)
    for n in "qkv":
        y[n][:, :, 4 * hw:] = inputs.bf16_bits(rng.standard_normal(y[n][:, :, 4 * hw:].shape).astype(np.float32))
    c = run_gpu(w, y)
    early = 2 * (w.grid_h // 8) * (w.grid_w // 8)
    assert np.array_equal(a["O"][:, :, :4 * hw], c["O"][:, :, :4 * hw])
    assert np.array_equal(a["lse"][:, :, :4 * hw], c["lse"][:, :, :4 * hw])
    assert np.array_equal(a["col_idx"][:, :, :a["row_ptr"][early]], c["col_idx"][:, :, :c["row_ptr"][early]])
    assert not np.array_equal(a["O"][:, :, 4 * hw:], c["O"][:, :, 4 * hw:])


def test_bad_tensors_raise():
    w = W.Workload("err", 1, 2, 128, 16, 24, 4, 0, 4, keep_ratio=0.5)
    p = lcsa.problem(w)
    x = inputs.make_inputs(w, 0)
    q, k, v = (to_device(x[n]) for n in "qkv")
    with pytest.raises(ValueError):
        lcsa.lcsa_pool(p, q.float(), k)
    with pytest.raises(ValueError):
        lcsa.lcsa_pool(p, q[:, :, :100], k)
    rp = torch.from_numpy(lcsa.lcsa_csr_layout(p)[3]).cuda()
    with pytest.raises(ValueError):
        lcsa.lcsa_score_select(p, torch.zeros(3, device="cuda"), torch.zeros(3, device="cuda"), rp)
    bad = lcsa.problem(w.replace(head_dim=80))
    with pytest.raises(lcsa.LcsaError):
        lcsa.lcsa_csr_layout(bad)
