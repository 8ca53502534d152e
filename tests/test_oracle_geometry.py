"""Pins for the oracle's geometry: visibility (block-causal + window), K_i and CSR sizes.

Every expectation here comes from something other than the oracle's own code: closed-form counts,
the window invariants that follow from the method's purpose (a bounded relative positional range at
any resolution; FlashVSR summary, sec. 2.3) and hand arithmetic on the workload shapes.
"""
import itertools

import numpy as np
import pytest

from block_sparse_causal_lcsa_amd import workloads as W
from oracle import lcsa_oracle as O


def small(**kw):
    base = dict(name="t", batch=1, heads=1, head_dim=16, grid_h=32, grid_w=48, kv_frames=4,
                q_frame0=0, q_frames=4, dtype="f32")
    base.update(kw)
    return W.Workload(**base)


# ---------------------------------------------------------------------------- causality
@pytest.mark.parametrize("q0,qf,kvf", [(0, 4, 4), (2, 2, 4), (4, 2, 6), (0, 2, 6)])
def test_block_causal_without_window(q0, qf, kvf):
    p = small(q_frame0=q0, q_frames=qf, kv_frames=kvf)
    vis = O.visible(p)
    qb, kb = O.query_blocks(p), O.key_blocks(p)
    for i, (ti, _, _) in enumerate(qb):
        for j, (tj, _, _) in enumerate(kb):
            assert vis[i, j] == (tj <= ti)
    # every query block sees at least its own spatial block in its own temporal block
    assert vis.sum(axis=1).min() >= 1


# ------------------------------------------------------------------------ window invariants
def trunc_count(c, n, r):
    return min(c + r, n - 1) - max(c - r, 0) + 1


@pytest.mark.parametrize("n,wb", list(itertools.product([5, 6, 9, 11, 12, 21], [1, 3, 9, 13, 41])))
def test_window_axis_invariants(n, wb):
    r = (wb - 1) // 2
    for c in range(n):
        tr = O.window_blocks(O.WIN_TRUNCATED, c, n, wb)
        pr = O.window_blocks(O.WIN_PRESERVING, c, n, wb)
        # W2: truncated = blocks within r of c, clipped to the frame
        assert len(tr) == trunc_count(c, n, r)
        assert c in tr and c in pr
        assert all(abs(x - c) <= r for x in tr)
        # W3: preserving keeps exactly wb contiguous blocks when the axis has that many
        assert len(pr) == min(wb, n)
        assert max(pr) - min(pr) + 1 == len(pr)
        # W4: truncated is a subset; equal for interior queries
        assert tr <= pr
        if r <= c <= n - 1 - r:
            assert tr == pr
        # W1 (per axis): any two tokens of the two blocks differ by < wb*8 tokens
        assert all(abs(x - c) * 8 + 7 < wb * 8 for x in pr)
        # W6: translation equivariance in the interior
        if r <= c and c + 1 <= n - 1 - r:
            assert O.window_blocks(O.WIN_TRUNCATED, c + 1, n, wb) == {x + 1 for x in tr}
    # W2 symmetry of the truncated relation
    for a in range(n):
        for b in range(n):
            assert (b in O.window_blocks(O.WIN_TRUNCATED, a, n, wb)) == \
                   (a in O.window_blocks(O.WIN_TRUNCATED, b, n, wb))
    # W5: a window at least 2n-1 blocks wide is no window
    if wb >= 2 * n - 1:
        for c in range(n):
            assert O.window_blocks(O.WIN_TRUNCATED, c, n, wb) == set(range(n))
            assert O.window_blocks(O.WIN_PRESERVING, c, n, wb) == set(range(n))


@pytest.mark.parametrize("mode", [O.WIN_TRUNCATED, O.WIN_PRESERVING])
def test_window_in_time_and_token_range(mode):
    # 40x56 grid -> 5x7 blocks; window 24 tokens -> 3 blocks
    p = small(grid_h=40, grid_w=56, kv_frames=6, q_frame0=2, q_frames=4, win_mode=mode, win_h=24, win_w=24)
    vis = O.visible(p)
    qb, kb = O.query_blocks(p), O.key_blocks(p)
    Hb, Wb = 5, 7
    for i, (ti, hi, wi) in enumerate(qb):
        sets = []
        for tb in range(p.kv_frames // 2):
            s = {(hj, wj) for j, (tj, hj, wj) in enumerate(kb) if tj == tb and vis[i, j]}
            if tb <= ti:
                sets.append(s)
            else:
                assert s == set()            # causality still holds with a window
        # W7: the same spatial window in every visible temporal block
        assert all(s == sets[0] for s in sets)
        # W1: every attended token pair is less than win tokens apart on each axis
        for (hj, wj) in sets[0]:
            assert abs(hj - hi) * 8 + 7 < p.win_h and abs(wj - wi) * 8 + 7 < p.win_w
        if mode == O.WIN_PRESERVING:
            assert len(sets[0]) == 9
        else:
            assert len(sets[0]) == trunc_count(hi, Hb, 1) * trunc_count(wi, Wb, 1)


# ------------------------------------------------------------------------------- K_i rule
def test_keep_count_rule():
    for rho in [0.01, 0.05, 0.136, 0.25, 0.5, 0.9, 1.0]:
        p = small(keep_ratio=rho)
        for n in range(1, 900):
            k = O.keep_count(p, n)
            assert 1 <= k <= n
            if rho * n >= 0.5:
                assert abs(k / n - rho) <= 0.5 / n + 1e-12
    p = small(keep_ratio=0.136)
    assert O.keep_count(p, 198) == 27          # 26.928 rounds to 27
    assert [O.keep_count(p, n) for n in (66, 132, 198, 264)] == [9, 18, 27, 36]
    p = small(topk=3)
    assert [O.keep_count(p, n) for n in (1, 2, 3, 4, 8)] == [1, 2, 3, 3, 3]


# ------------------------------------------------------------------- workload-level sizes
def _load_golden():
    rows = {}
    with open(__file__.replace("test_oracle_geometry.py", "golden/workload_sizes.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            name, nqb, nkb, nnz, kmin, kmax = line.split()
            rows[name] = tuple(int(x) for x in (nqb, nkb, nnz, kmin, kmax))
    return rows


@pytest.mark.parametrize("w", W.ALL, ids=lambda w: w.name)
def test_workload_sizes(w):
    """nqb, nkb, nnz per head and the K_i range match hand-derived values (tests/golden)."""
    golden = _load_golden()[w.name]
    vis = O.visible(w)
    rp = O.csr_row_ptr(w, vis)
    k = np.diff(rp)
    assert (vis.shape[0], vis.shape[1], int(rp[-1]), int(k.min()), int(k.max())) == golden
