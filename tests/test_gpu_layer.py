"""GPU tests of the DiT attention layer around LCSA (row f4): lcsa_rope_qkv against the oracle's
rope_3d, and every stage of DitLcsaLayer.step against the oracle given the previous stage's GPU
output (the two projections are library GEMMs and are checked within bf16 GEMM rounding).

RoPE bound: the kernel rounds an fp32 rotation of the bf16 input once to bf16 (8 significant bits:
half an ulp is at most 2^-8 of the value), so per element
|gpu - ref| <= 2^-8 |ref| + (2^-22 a_max + 2^-20) |pair|, with ref the fp64 rotation of the same bf16
input, |pair| the norm of the element's rotation pair and a_max the largest angle (the largest
position: frequencies are <= 1): the fp32 angle pos * freq is off by about 2^-23 of itself, sin/cos and
the rotation by a few fp32 ulps. v is copied bit for bit.
"""
import numpy as np
import pytest
import torch

from block_sparse_causal_lcsa_amd import inputs, lcsa
from block_sparse_causal_lcsa_amd import workloads as W
from block_sparse_causal_lcsa_amd.layer import DitLcsaLayer
from oracle import lcsa_oracle as O

from parity import check_attention, from_device

pytestmark = pytest.mark.gpu


def bf16_rand(shape, seed, scale=1.0):
    x = np.random.default_rng(seed).standard_normal(shape).astype(np.float32) * np.float32(scale)
    bits = inputs.bf16_bits(x)
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda(), inputs.to_f64(bits)


def check_rope(got, ref, x64, a_max):
    pair = np.sqrt(x64[..., 0::2] ** 2 + x64[..., 1::2] ** 2)
    pair = np.repeat(pair, 2, axis=-1)
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + (2.0 ** -22 * a_max + 2.0 ** -20) * pair
    assert np.all(err <= bound), float((err - bound).max())
    return float(err.max())


@pytest.mark.parametrize("grid,heads,d,dims,frame0,frames", [
    ((21, 37), 2, 128, (44, 42, 42), 6, 2),
    ((16, 24), 3, 64, (22, 20, 22), 0, 4),
    ((48, 88), 12, 128, (44, 42, 42), 40, 2),
])
def test_rope_matches_oracle(grid, heads, d, dims, frame0, frames):
    w = W.Workload("rope", 2, heads, d, grid[0], grid[1], frames, 0, frames)
    p = lcsa.problem(w)
    n = frames * grid[0] * grid[1]
    qkv, qkv64 = bf16_rand((2, n, 3 * heads * d), 11, 2.0)
    rope = lcsa.LcsaRope(*dims, 10000.0)
    q, k, v = lcsa.lcsa_rope_qkv(p, rope, qkv, frame0)
    torch.cuda.synchronize()
    x = qkv64.reshape(2, n, 3, heads, d).transpose(2, 0, 3, 1, 4)   # [3, B, heads, N, d]
    for got, src in ((q, x[0]), (k, x[1])):
        check_rope(from_device(got), O.rope_3d(w, src, frame0, dims, 10000.0), src,
                   max(frame0 + frames, grid[0], grid[1]))
    assert np.array_equal(from_device(v), x[2])


def test_layer_stages_against_oracle():
    chunk = W.Workload("layer_24x40", 1, 2, 128, 24, 40, 2, 0, 2, keep_ratio=0.4)
    p = lcsa.problem(chunk)
    layer = DitLcsaLayer(p, cache_tblocks=2, seed=3)
    N, C = 2 * 24 * 40, 256
    w_qkv = from_device(layer.w_qkv)
    w_o = from_device(layer.w_o)
    for c in range(4):
        x, x64 = bf16_rand((1, N, C), 100 + c)
        out, res = layer.step(x)
        torch.cuda.synchronize()
        # projection (library GEMM, bf16 output): within bf16 rounding of the fp64 product
        qkv = from_device(res["qkv"])
        ref = x64[0] @ w_qkv
        assert np.abs(qkv[0] - ref).max() <= 2.0 ** -7 * np.abs(ref).max()
        # RoPE of the GPU's qkv
        xs = qkv.reshape(1, N, 3, 2, 128).transpose(2, 0, 3, 1, 4)
        q64 = O.rope_3d(chunk, xs[0], 2 * c, (44, 42, 42), 10000.0)
        check_rope(from_device(res["q"]), q64, xs[0], 40)
        pw, kw, vw, _ = layer.stream.window()
        kw64, vw64 = from_device(kw), from_device(vw)
        k_new = O.rope_3d(chunk, xs[1], 2 * c, (44, 42, 42), 10000.0)
        check_rope(kw64[:, :, -N:], k_new, xs[1], 40)
        assert np.array_equal(vw64[:, :, -N:], xs[2])
        # LCSA on the GPU's q and window K/V: selection and attention against the oracle
        q_gpu = from_device(res["q"])
        want = O.forward(pw, q_gpu, kw64, vw64)
        col = res["col_idx"].cpu().numpy().astype(np.int64)
        assert np.mean(col == want["col_idx"]) > 0.99
        gpu = dict(row_ptr=res["row_ptr"].cpu().numpy().astype(np.int64), col_idx=col,
                   O=from_device(res["o"]), lse=res["lse"].cpu().numpy().astype(np.float64))
        check_attention(pw, (q_gpu, kw64, vw64), gpu)
        # output projection of the GPU's O
        o_tok = from_device(res["o_tokens"]).reshape(N, C)
        ref_out = o_tok @ w_o
        assert np.abs(from_device(out)[0] - ref_out).max() <= 2.0 ** -7 * np.abs(ref_out).max() + 1e-3


def test_layer_chunk_768x1408_lcsa_matches_direct_calls():
    """At the 768x1408 chunk shape (12 heads, d 128): the layer's LCSA output equals lcsa.forward on
    contiguous copies of its window, bit for bit, over 4 chunks (cache 3)."""
    w = W.CHUNK_768
    chunk = w.replace(kv_frames=2, q_frame0=0, q_frames=2)
    layer = DitLcsaLayer(lcsa.problem(chunk), cache_tblocks=3, seed=5)
    N, C = 2 * 48 * 88, 12 * 128
    for c in range(4):
        x, _ = bf16_rand((1, N, C), 200 + c)
        out, res = layer.step(x)
        pw, kw, vw, _ = layer.stream.window()
        ref = lcsa.forward(pw, res["q"], kw.contiguous(), vw.contiguous())
        torch.cuda.synchronize()
        assert torch.equal(ref["col_idx"], res["col_idx"]) and torch.equal(ref["o"], res["o"].contiguous())
        assert torch.isfinite(out.float()).all()
