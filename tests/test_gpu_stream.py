"""GPU tests of the streaming state (lcsa_stream_*): chunk-by-chunk LCSA through the K/V rings and
the pooled-K cache.

Each chunk pushes one temporal block of K/V and runs pool(q) -> score_select -> attn_fwd on the
window the state describes. The result must equal, bit for bit, the same three calls on K/V of the
window's blocks laid out contiguously (the rings and the cached pooled K change only where the data
sits, not the arithmetic), and the pooled-K window must equal lcsa_pool of that K. On small
sequences the chunk is also checked against the oracle's stream_forward (selection bit-exact up to
near-ties, attention within the forward's tolerances).
"""
import numpy as np
import pytest
import torch

from block_sparse_causal_lcsa_amd import inputs, lcsa
from block_sparse_causal_lcsa_amd import workloads as W
from oracle import lcsa_oracle as O

from parity import check_attention, from_device, to_device

pytestmark = pytest.mark.gpu


def run_stream(seq, cache, seed=0, oracle_chunks=(), ring=0, in_place=()):
    """Streams every temporal block of `seq`; chunks in `in_place` are written into the reserved slot
    by the caller (torch copy) and pushed from there (no library copy)."""
    chunk = seq.replace(kv_frames=2, q_frame0=0, q_frames=2)
    p = lcsa.problem(chunk)
    x = inputs.make_inputs(seq, seed)
    q, k, v = (to_device(x[n]) for n in "qkv")
    tbt = 2 * seq.grid_h * seq.grid_w
    s = lcsa.Stream(p, cache, ring)
    nchunks = seq.kv_frames // 2
    x64 = [inputs.to_f64(x[n]) for n in "qkv"] if oracle_chunks else None
    for c in range(nchunks):
        rows = slice(c * tbt, (c + 1) * tbt)
        if c in in_place:
            ks, vs = s.reserve()
            ks.copy_(k[:, :, rows])
            vs.copy_(v[:, :, rows])
            s.push(ks, vs)
        else:
            s.push(k[:, :, rows], v[:, :, rows])
        out = s.forward(q[:, :, rows])
        first = max(0, c - cache + 1)
        win = slice(first * tbt, (c + 1) * tbt)
        pw = out["problem"]
        assert (pw.kv_frames, pw.q_frame0) == (2 * (c - first + 1), 2 * (c - first))
        kw, vw = k[:, :, win].contiguous(), v[:, :, win].contiguous()
        ref = lcsa.forward(pw, q[:, :, rows].contiguous(), kw, vw)
        torch.cuda.synchronize()
        for name in ("q_pooled", "k_pooled", "col_idx", "o", "lse"):
            assert torch.equal(out[name], ref[name]), (c, name)
        if c in oracle_chunks:
            want = O.stream_forward(chunk, *x64, cache_tblocks=cache, chunks=[c])[c]
            gpu = dict(row_ptr=ref["row_ptr"].cpu().numpy().astype(np.int64),
                       col_idx=out["col_idx"].cpu().numpy().astype(np.int64), O=from_device(out["o"]),
                       lse=out["lse"].cpu().numpy().astype(np.float64))
            _, pwo = O.stream_window(chunk, c, cache)
            assert np.array_equal(gpu["row_ptr"], want["row_ptr"])
            assert np.array_equal(out["k_pooled"].cpu().numpy(), want["kbar"].astype(np.float32))
            same = np.mean(gpu["col_idx"] == want["col_idx"])
            assert same > 0.99, same
            qw = x64[0][:, :, rows]
            check_attention(pwo, (qw, x64[1][:, :, win], x64[2][:, :, win]), gpu)
    assert s.state.held == min(nchunks, cache) and s.state.pushed == nchunks


def test_stream_small_bf16_cache3():
    """Minimal ring (5 slots): compaction after the 5th and 8th push; chunks 3 and 6 pushed in place."""
    seq = W.Workload("stream_24x40_t20", 1, 2, 128, 24, 40, 20, 0, 20, keep_ratio=0.4)
    run_stream(seq, 3, oracle_chunks=(0, 2, 5, 9), in_place=(3, 6))


def test_stream_large_ring():
    seq = W.Workload("stream_16x24_t12", 1, 3, 128, 16, 24, 12, 0, 12, keep_ratio=0.3)
    run_stream(seq, 2, seed=3, ring=6, in_place=(0, 1, 2, 5))


def test_stream_small_f32_d64_window_cache2():
    seq = W.Workload("stream_24x32_t8_f32", 2, 2, 64, 24, 32, 8, 0, 8, dtype="f32", win_mode=1, win_h=24,
                     win_w=24, keep_ratio=0.5)
    run_stream(seq, 2, seed=1, oracle_chunks=(3,), in_place=(2,))


def test_stream_ragged_grid():
    """A 21x37 grid (partial last block row and column) streamed through a 2-block cache."""
    seq = W.Workload("stream_21x37_t8", 1, 2, 128, 21, 37, 8, 0, 8, keep_ratio=0.4)
    run_stream(seq, 2, seed=4, oracle_chunks=(2,), in_place=(1,))


def test_stream_cache1():
    seq = W.Workload("stream_16x24_t6_c1", 1, 2, 128, 16, 24, 6, 0, 6, topk=2)
    run_stream(seq, 1, seed=2, oracle_chunks=(1,), in_place=(2,))


def test_stream_chunk_768x1408():
    """The 768x1408 chunk shape (12 heads, d 128, 13.6% kept) over 5 chunks with the 3-block cache of
    the benchmark workload: bitwise equal to the direct calls on every chunk."""
    seq = W.CHUNK_768.replace(kv_frames=10, q_frame0=0, q_frames=10)
    run_stream(seq, 3)
