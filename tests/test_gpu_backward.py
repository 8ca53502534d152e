"""GPU parity of lcsa_attn_bwd (gradients of the block-sparse attention for a fixed selection)
against the oracle's fp64 attend_bwd, through the C ABI.

The forward runs on the GPU (pool -> select -> attn_fwd); its selection, O and lse feed the
backward, and the oracle recomputes the exact gradients for the same selection from the same bf16
Q, K, V and dO.

Tolerance. The kernels round P (for dV) and dS (for dK, dQ) to bf16 before the second products and
take Delta = rowsum(dO * O) from the bf16 O; everything else is fp32 accumulation of exact bf16
products. Replaying exactly those roundings on the CPU gives a normalised error of about 0.3%
(max |d| / max |ref| and mean |d| / mean |ref| between 0.13% and 0.36% on 24x40 and 24x32 grids,
d = 64 and 128). The bar is 1% for both ratios, per gradient tensor.

At full chunk size dQ is compared on sampled query blocks, and dK/dV on sampled key blocks with the
oracle run over every query block that kept them (so those rows are complete); key blocks nobody
kept must be exactly zero, and two calls must agree bit for bit (no atomics).
"""
import json
import sys

import numpy as np
import pytest
import torch

from block_sparse_causal_lcsa_amd import inputs, lcsa
from block_sparse_causal_lcsa_amd import workloads as W
from oracle import lcsa_oracle as O

from parity import from_device, to_device

pytestmark = pytest.mark.gpu

REL_MAX, REL_MEAN = 1e-2, 1e-2


def run(w, seed, negate_k=False):
    p = lcsa.problem(w)
    x = inputs.make_inputs(w, seed)
    if negate_k:
        x["k"] = x["k"] ^ np.uint16(0x8000)   # bf16 sign bit
    g = inputs.make_grad(w, seed)
    q, k, v, d_o = (to_device(a) for a in (x["q"], x["k"], x["v"], g))
    out = lcsa.forward(p, q, k, v)
    dq, dk, dv = lcsa.lcsa_attn_bwd(p, q, k, v, out["o"], d_o, out["lse"], out["row_ptr"], out["col_idx"])
    dq2, dk2, dv2 = lcsa.lcsa_attn_bwd(p, q, k, v, out["o"], d_o, out["lse"], out["row_ptr"], out["col_idx"])
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2), "backward not deterministic"
    x64 = [inputs.to_f64(x[n]) for n in "qkv"]
    return dict(x64=x64, g64=inputs.to_f64(g), row_ptr=out["row_ptr"].cpu().numpy().astype(np.int64),
                col=out["col_idx"].cpu().numpy().astype(np.int64),
                dq=from_device(dq), dk=from_device(dk), dv=from_device(dv))


def compare(name, got, ref, mask):
    d = np.abs(got[mask] - ref[mask])
    r = np.abs(ref[mask])
    assert np.all(np.isfinite(got[mask])), f"{name}: non-finite gradient"
    stats = dict(max_abs=float(d.max()), mean_abs=float(d.mean()), rel_max=float(d.max() / r.max()),
                 rel_mean=float(d.mean() / r.mean()))
    assert stats["rel_max"] <= REL_MAX and stats["rel_mean"] <= REL_MEAN, (name, stats)
    return stats


def kept_columns(w, rp, col):
    """Per (b, h): boolean [nkb], key block kept by at least one query block."""
    out = np.zeros((w.batch, w.heads, w.nkb), dtype=bool)
    for b in range(w.batch):
        for h in range(w.heads):
            c = col[b, h]
            out[b, h, c[(c >= 0) & (c < w.nkb)]] = True
    return out


def token_mask(w, blocks_per_bh, which):
    """[B, Hh, N] token mask of the given blocks per (b, h)."""
    f0 = w.q_frame0 if which == "q" else 0
    blk = O.query_blocks(w) if which == "q" else O.key_blocks(w)
    n = (w.q_frames if which == "q" else w.kv_frames) * w.grid_h * w.grid_w
    m = np.zeros((w.batch, w.heads, n), dtype=bool)
    for (b, h), bl in blocks_per_bh.items():
        for j in bl:
            m[b, h, O.block_tokens(w, blk[j], f0)] = True
    return m


def check_unkept_zero(w, r):
    """Key blocks no query block kept get exactly zero dK and dV; returns how many there were."""
    kept = kept_columns(w, r["row_ptr"], r["col"])
    unkept = {(b, h): np.flatnonzero(~kept[b, h]).tolist() for b in range(w.batch) for h in range(w.heads)}
    mz = token_mask(w, unkept, "k")
    assert not np.any(r["dk"][mz]) and not np.any(r["dv"][mz])
    return int((~kept).sum())


def report(name, stats):
    print(f"PARITY-BWD {name} {json.dumps(stats)}", flush=True)
    sys.stdout.flush()


SMALL = [
    W.Workload("bwd_24x40_q2of4", 1, 2, 128, 24, 40, 4, 2, 2, keep_ratio=0.4),
    W.Workload("bwd_24x40_q2of4_win_trunc", 1, 1, 128, 24, 40, 4, 2, 2, win_mode=1, win_h=24, win_w=24,
               keep_ratio=0.5),
    W.Workload("bwd_24x32_all6_d64", 1, 2, 64, 24, 32, 6, 0, 6, keep_ratio=0.3),
    W.Workload("bwd_16x24_b2_pres_topk3", 2, 2, 128, 16, 24, 4, 0, 4, win_mode=2, win_h=8, win_w=24, topk=3),
    W.Workload("bwd_8x8_one_block", 1, 1, 64, 8, 8, 2, 0, 2, keep_ratio=1.0),
    W.Workload("bwd_16x40_topk1", 1, 2, 128, 16, 40, 6, 4, 2, topk=1),
    # grids that are not multiples of 8: partial edge blocks
    W.Workload("bwd_ragged_21x37", 1, 2, 128, 21, 37, 4, 2, 2, keep_ratio=0.4),
    W.Workload("bwd_ragged_13x10_d64_pres", 1, 2, 64, 13, 10, 4, 0, 4, win_mode=2, win_h=24, win_w=24,
               keep_ratio=0.5),
    W.Workload("bwd_ragged_3x5", 1, 1, 128, 3, 5, 6, 4, 2, topk=2),
    # token-granular windows (the last: one kept block per row under a 3x3 window)
    W.Workload("bwd_tokwin_trunc_24x40_w13x17", 1, 2, 128, 24, 40, 4, 2, 2, win_mode=3, win_h=13, win_w=17,
               keep_ratio=0.5),
    W.Workload("bwd_tokwin_pres_21x37_w20x9", 1, 2, 128, 21, 37, 6, 4, 2, win_mode=4, win_h=20, win_w=9,
               keep_ratio=0.4),
    W.Workload("bwd_tokwin_w3_topk1", 1, 2, 64, 24, 32, 4, 2, 2, win_mode=3, win_h=3, win_w=3, topk=1),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_backward_small(w):
    r = run(w, 0)
    q, k, v = r["x64"]
    dQ, dK, dV = O.attend_bwd(w, q, k, v, r["row_ptr"], r["col"], r["g64"])
    allq = np.ones(dQ.shape[:3], dtype=bool)
    allk = np.ones(dK.shape[:3], dtype=bool)
    stats = {n: compare(n, r[n], ref, m) for n, ref, m in
             (("dq", dQ, allq), ("dk", dK, allk), ("dv", dV, allk))}
    stats["unkept_key_blocks"] = check_unkept_zero(w, r)
    if w.topk == 1:
        assert stats["unkept_key_blocks"] > 0
    report(w.name, stats)


def test_backward_rows_without_keys():
    """Token window 3x3, one kept block per row, K negated so the kept block is a neighbour: most
    query tokens see no kept key (forward O = 0, lse = -inf) and must get exactly zero dQ; the
    others, and dK / dV, meet the usual bar."""
    w = W.Workload("bwd_tokwin_blind_24x32_w3_topk1", 1, 2, 128, 24, 32, 4, 2, 2, win_mode=3, win_h=3, win_w=3,
                   topk=1)
    r = run(w, 0, negate_k=True)
    q, k, v = r["x64"]
    dQ, dK, dV = O.attend_bwd(w, q, k, v, r["row_ptr"], r["col"], r["g64"])
    blind = np.all(dQ == 0.0, axis=-1)
    assert blind.sum() > 0 and not np.any(r["dq"][blind])
    mk = np.ones(dK.shape[:3], dtype=bool)
    report(w.name, {"blind_rows": int(blind.sum()), "dq": compare("dq", r["dq"], dQ, ~blind),
                    "dk": compare("dk", r["dk"], dK, mk), "dv": compare("dv", r["dv"], dV, mk)})


def test_backward_full_selection_matches_dense():
    """keep ratio 1: the gradients equal those of dense block-causal attention (oracle's attend_bwd
    with every visible block, itself pinned to autograd of dense masked attention)."""
    w = W.Workload("bwd_dense_24x32", 1, 2, 128, 24, 32, 4, 0, 4, keep_ratio=1.0)
    r = run(w, 1)
    q, k, v = r["x64"]
    vis = O.visible(w)
    rp = np.concatenate([[0], np.cumsum(vis.sum(1))]).astype(np.int64)
    col = np.broadcast_to(np.concatenate([np.flatnonzero(vis[i]) for i in range(w.nqb)]),
                          (w.batch, w.heads, rp[-1]))
    assert np.array_equal(r["row_ptr"], rp) and np.array_equal(r["col"], col)
    dQ, dK, dV = O.attend_bwd(w, q, k, v, rp, col, r["g64"])
    m = np.ones(dQ.shape[:3], dtype=bool)
    mk = np.ones(dK.shape[:3], dtype=bool)
    report(w.name, {"dq": compare("dq", r["dq"], dQ, m), "dk": compare("dk", r["dk"], dK, mk),
                    "dv": compare("dv", r["dv"], dV, mk)})


def test_backward_chunk_768x1408_sampled():
    """The 768x1408 streaming chunk (12 heads, d = 128, 13.6% kept) at full size, sampled."""
    w = W.CHUNK_768
    r = run(w, 0)
    q, k, v = r["x64"]
    rp, col = r["row_ptr"], r["col"]
    rng = np.random.default_rng(7)
    heads = [(0, 0), (0, 5), (0, 11)]
    kept = kept_columns(w, rp, col)
    stats = {}
    # dQ on sampled query blocks
    qbl = sorted({0, w.nqb - 1} | set(rng.choice(w.nqb, 6, replace=False).tolist()))
    dQ, _, _ = O.attend_bwd(w, q, k, v, rp, col, r["g64"], qblocks=qbl, bh=heads)
    stats["dq"] = compare("dq", r["dq"], dQ, token_mask(w, {bh: qbl for bh in heads}, "q"))
    # dK, dV on sampled key blocks, oracle over every query block that kept them
    for b, h in heads:
        cand = np.flatnonzero(kept[b, h])
        js = sorted(set(rng.choice(cand, 3, replace=False).tolist()))
        rows = sorted({i for i in range(w.nqb) for j in js if j in col[b, h, rp[i]:rp[i + 1]]})
        _, dK, dV = O.attend_bwd(w, q, k, v, rp, col, r["g64"], qblocks=rows, bh=[(b, h)])
        m = token_mask(w, {(b, h): js}, "k")
        stats[f"dk_h{h}"] = compare("dk", r["dk"], dK, m)
        stats[f"dv_h{h}"] = compare("dv", r["dv"], dV, m)
    stats["unkept_key_blocks"] = check_unkept_zero(w, r)
    report(w.name, stats)


def test_backward_strided_inputs_match_contiguous():
    """Q, K, V, O and dO as [B, tokens, heads, d] storage viewed as [B, heads, tokens, d] (token
    stride heads*d): the gradients equal those of contiguous copies bit for bit."""
    w = W.Workload("bwd_strided", 2, 3, 128, 16, 24, 4, 2, 2, keep_ratio=0.5)
    p = lcsa.problem(w)
    x = inputs.make_inputs(w, 6)
    g = inputs.make_grad(w, 6)
    q, k, v, d_o = (to_device(a) for a in (x["q"], x["k"], x["v"], g))
    out = lcsa.forward(p, q, k, v)
    args = (out["row_ptr"], out["col_idx"])
    ref = lcsa.lcsa_attn_bwd(p, q, k, v, out["o"], d_o, out["lse"], *args)

    def strided(t):
        s = t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
        assert s.stride(2) == w.heads * w.head_dim and torch.equal(s, t)
        return s

    got = lcsa.lcsa_attn_bwd(p, strided(q), strided(k), strided(v), strided(out["o"]), strided(d_o), out["lse"],
                             *args)
    torch.cuda.synchronize()
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), name
