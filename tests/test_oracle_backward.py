"""Pins for the oracle's attention backward (gradients for a fixed selection).

Anchors: with every visible block kept the gradients must equal torch autograd of dense attention
under the block visibility mask (fp64, CPU); for a sparse selection the analytic gradients must
match central finite differences of the oracle's own forward; closed forms (zero upstream gradient,
keys that differ by a constant vector, constant upstream gradient for dV) complete the pins.
"""
import numpy as np
import pytest
import torch

from oracle import lcsa_oracle as O

from test_oracle_attention import rand_qkv, small, token_block_map


def full_selection(p):
    vis = O.visible(p)
    rp = O.csr_row_ptr(p, vis)
    nq = len(O.query_blocks(p))
    col = np.concatenate([np.flatnonzero(vis[i]) for i in range(nq)])
    return rp, np.broadcast_to(col, (p.batch, p.heads, col.size)).copy()


@pytest.mark.parametrize("mode", [O.WIN_NONE, O.WIN_TRUNCATED])
def test_full_selection_matches_autograd(mode):
    p = small(win_mode=mode, win_h=8 if mode else 0, win_w=8 if mode else 0, grid_w=24, heads=2)
    q, k, v = rand_qkv(p, seed=4)
    rng = np.random.default_rng(5)
    dO = rng.standard_normal(q.shape)
    rp, col = full_selection(p)
    dQ, dK, dV = O.attend_bwd(p, q, k, v, rp, col, dO)
    qmap, kmap = token_block_map(p)
    vis = O.visible(p)
    mask = torch.from_numpy(vis[qmap][:, kmap])
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=p.scale)
    out.backward(torch.from_numpy(dO))
    for got, want in ((dQ, tq.grad), (dK, tk.grad), (dV, tv.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-10, atol=1e-11)


def test_finite_differences_sparse_selection():
    p = small(keep_ratio=0.4, heads=1, grid_h=16, grid_w=16)
    q, k, v = rand_qkv(p, seed=7)
    rng = np.random.default_rng(8)
    G = rng.standard_normal(q.shape)
    # a fixed sparse selection: the oracle's own, from these inputs
    fw = O.forward(p, q, k, v)
    rp, col = fw["row_ptr"], fw["col_idx"]
    assert rp[-1] < O.visible(p).sum()  # really sparse
    dQ, dK, dV = O.attend_bwd(p, q, k, v, rp, col, G)

    def loss(q_, k_, v_):
        out, _ = O.attend(p, q_, k_, v_, rp, col)
        return float((out * G).sum())

    eps = 1e-6
    for which, grad in (("q", dQ), ("k", dK), ("v", dV)):
        d = rng.standard_normal(q.shape if which == "q" else k.shape)
        args_p = {"q": q, "k": k, "v": v}
        args_m = dict(args_p)
        args_p[which] = args_p[which] + eps * d
        args_m[which] = args_m[which] - eps * d
        fd = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
        an = float((grad * d).sum())
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (which, fd, an)


def test_closed_forms():
    p = small(keep_ratio=0.5, heads=1)
    q, k, v = rand_qkv(p, seed=9)
    fw = O.forward(p, q, k, v)
    rp, col = fw["row_ptr"], fw["col_idx"]
    # zero upstream gradient: zero gradients
    z = O.attend_bwd(p, q, k, v, rp, col, np.zeros_like(q))
    for g in z:
        assert np.all(g == 0)
    # keys shifted by one constant vector: softmax is unchanged, so dQ is unchanged
    rng = np.random.default_rng(10)
    dO = rng.standard_normal(q.shape)
    dQ0, _, _ = O.attend_bwd(p, q, k, v, rp, col, dO)
    dQ1, _, _ = O.attend_bwd(p, q, k + rng.standard_normal(k.shape[-1]), v, rp, col, dO)
    np.testing.assert_allclose(dQ1, dQ0, rtol=1e-9, atol=1e-10)
    # constant upstream gradient c: dV of a key token is c times the total probability it received
    c = rng.standard_normal(q.shape[-1])
    _, _, dV = O.attend_bwd(p, q, k, v, rp, col, np.broadcast_to(c, q.shape).copy())
    mass = np.zeros(k.shape[2])
    qb, kb = O.query_blocks(p), O.key_blocks(p)
    for i in range(len(qb)):
        qt = O.block_tokens(p, qb[i], p.q_frame0)
        kt = np.concatenate([O.block_tokens(p, kb[j], 0) for j in col[0, 0, rp[i]:rp[i + 1]]])
        lg = p.scale * (q[0, 0, qt] @ k[0, 0, kt].T)
        P = np.exp(lg - lg.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        mass[kt] += P.sum(axis=0)
    np.testing.assert_allclose(dV[0, 0], mass[:, None] * c[None, :], rtol=1e-10, atol=1e-12)
