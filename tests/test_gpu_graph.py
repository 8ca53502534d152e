"""The three calls captured into one HIP graph (as the benchmark replays them) give, on every replay,
exactly the outputs of eager launches on the same inputs, with unrelated eager work and
synchronisations between the replays."""
import numpy as np
import pytest
import torch

from block_sparse_causal_lcsa_amd import inputs, lcsa
from block_sparse_causal_lcsa_amd import workloads as W

from parity import to_device

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("w", [W.CHUNK_768, W.UHD_TRUNC], ids=lambda w: w.name)
def test_graph_replay_matches_eager(w):
    p = lcsa.problem(w)
    x = inputs.make_inputs(w, seed=3)
    dev = torch.device("cuda:0")
    q, k, v = (to_device(x[n], dev) for n in "qkv")
    nqb, nkb, nnz, rp = lcsa.lcsa_csr_layout(p)
    row_ptr = torch.from_numpy(rp).to(dev)
    qp = torch.empty((w.batch, w.heads, nqb, w.head_dim), dtype=torch.float32, device=dev)
    kp = torch.empty((w.batch, w.heads, nkb, w.head_dim), dtype=torch.float32, device=dev)
    col = torch.empty((w.batch, w.heads, nnz), dtype=torch.int32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.batch, w.heads, w.nq_tokens), dtype=torch.float32, device=dev)

    def step():
        s = torch.cuda.current_stream()
        lcsa.lcsa_pool(p, q, k, qp, kp, stream=s)
        lcsa.lcsa_score_select(p, qp, kp, row_ptr, col, stream=s)
        lcsa.lcsa_attn_fwd(p, q, k, v, row_ptr, col, o, lse, stream=s)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (qp, kp, col, o, lse)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()

    # unrelated eager work between replays: another forward on a perturbed copy of the inputs
    q2 = (q.float() * 0.5).to(q.dtype)
    for r in range(4):
        for t in (qp, kp, o, lse):
            t.fill_(float("nan"))
        col.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        other = lcsa.forward(p, q2, k, v, row_ptr=row_ptr)
        torch.cuda.synchronize()
        for name, got, want in zip(("q_pooled", "k_pooled", "col_idx", "o", "lse"), (qp, kp, col, o, lse), ref):
            assert torch.equal(got, want), f"replay {r}: {name} differs from the eager launch"
        assert other["o"].shape == o.shape


def test_backward_graph_replay_matches_eager():
    """lcsa_attn_bwd (delta, CSC transpose, dQ, dK/dV launches; caller-owned workspace) captured into
    a graph: every replay equals the eager call bit for bit, with a different eager backward between
    replays reusing nothing but the library."""
    w = W.Workload("graph_bwd", 1, 4, 128, 24, 40, 4, 2, 2, keep_ratio=0.4)
    p = lcsa.problem(w)
    x = inputs.make_inputs(w, seed=8)
    g = inputs.make_grad(w, seed=8)
    dev = torch.device("cuda:0")
    q, k, v, d_o = (to_device(a, dev) for a in (x["q"], x["k"], x["v"], g))
    out = lcsa.forward(p, q, k, v)
    ws = torch.empty(lcsa.lcsa_attn_bwd_workspace_size(p), dtype=torch.uint8, device=dev)
    grads = [torch.empty((w.batch, w.heads, n, w.head_dim), dtype=torch.float32, device=dev)
             for n in (w.nq_tokens, w.nk_tokens, w.nk_tokens)]
    args = (p, q, k, v, out["o"], d_o, out["lse"], out["row_ptr"], out["col_idx"])

    def step():
        lcsa.lcsa_attn_bwd(*args, *grads, workspace=ws, stream=torch.cuda.current_stream())

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in grads]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    d_o2 = (d_o.float() * -2.0).to(d_o.dtype)
    for r in range(4):
        for t in grads:
            t.fill_(float("nan"))
        ws.fill_(255)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("dq", "dk", "dv"), grads, ref):
            assert torch.equal(got, want), f"replay {r}: {name} differs from the eager call"
        other = lcsa.lcsa_attn_bwd(p, q, k, v, out["o"], d_o2, out["lse"], out["row_ptr"], out["col_idx"])
        torch.cuda.synchronize()
        assert torch.isfinite(other[0]).all()
