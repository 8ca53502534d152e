"""Pins of the oracle's streaming reading (stream_forward): a chunk is the forward over the window of
cached temporal blocks plus the new one.

- With a cache long enough to hold the whole history, every chunk equals the rows of its temporal
  block in one forward over the whole sequence (block causality already hides the future, and the
  visible set, K_i, scores and selection of those rows are the same).
- With a short cache, blocks older than the window do not influence the chunk (perturbing them leaves
  it bitwise unchanged), while a block inside the window does.
- With a cache of one block, a chunk is the plain forward of its own two frames.
"""
import numpy as np

from block_sparse_causal_lcsa_amd import inputs
from block_sparse_causal_lcsa_amd import workloads as W
from oracle import lcsa_oracle as O

SEQ = W.Workload("stream_seq_16x24_t8", 1, 2, 64, 16, 24, 8, 0, 8, keep_ratio=0.3, dtype="f32")
CHUNK = SEQ.replace(kv_frames=2, q_frame0=0, q_frames=2)


def seq_inputs(seed=0):
    x = inputs.make_inputs(SEQ, seed)
    return [inputs.to_f64(x[n]) for n in "qkv"]


def test_full_cache_equals_whole_sequence_forward():
    q, k, v = seq_inputs()
    full = O.forward(SEQ, q, k, v)
    st = O.stream_forward(CHUNK, q, k, v, cache_tblocks=4)
    hw = SEQ.grid_h * SEQ.grid_w
    bpt = (SEQ.grid_h // 8) * (SEQ.grid_w // 8)
    for c, out in st.items():
        rows = slice(2 * c * hw, 2 * (c + 1) * hw)
        assert np.allclose(out["O"], full["O"][:, :, rows], rtol=0, atol=1e-12)
        assert np.allclose(out["lse"], full["lse"][:, :, rows], rtol=0, atol=1e-12)
        # the chunk's selected key blocks are the full forward's selection of those rows
        rp = full["row_ptr"]
        for i in range(bpt):
            gi = c * bpt + i
            want = full["col_idx"][:, :, rp[gi]:rp[gi + 1]]
            got = out["col_idx"][:, :, out["row_ptr"][i]:out["row_ptr"][i + 1]]
            assert np.array_equal(got, want)


def test_evicted_blocks_have_no_influence():
    q, k, v = seq_inputs(1)
    base = O.stream_forward(CHUNK, q, k, v, cache_tblocks=2, chunks=[3])[3]
    hw = SEQ.grid_h * SEQ.grid_w
    old = slice(0, 4 * hw)                 # temporal blocks 0 and 1: outside chunk 3's window {2, 3}
    k2, v2 = k.copy(), v.copy()
    k2[:, :, old] += 5.0
    v2[:, :, old] *= -3.0
    pert = O.stream_forward(CHUNK, q, k2, v2, cache_tblocks=2, chunks=[3])[3]
    assert np.array_equal(pert["O"], base["O"]) and np.array_equal(pert["col_idx"], base["col_idx"])
    inside = slice(4 * hw, 6 * hw)         # temporal block 2: inside the window
    v3 = v.copy()
    v3[:, :, inside] += 1.0
    moved = O.stream_forward(CHUNK, q, k, v3, cache_tblocks=2, chunks=[3])[3]
    assert not np.allclose(moved["O"], base["O"])


def test_cache_of_one_block_is_the_chunk_alone():
    q, k, v = seq_inputs(2)
    hw = SEQ.grid_h * SEQ.grid_w
    st = O.stream_forward(CHUNK, q, k, v, cache_tblocks=1, chunks=[2])[2]
    rows = slice(4 * hw, 6 * hw)
    alone = O.forward(CHUNK, q[:, :, rows], k[:, :, rows], v[:, :, rows])
    assert np.array_equal(st["O"], alone["O"]) and np.array_equal(st["lse"], alone["lse"])


def test_window_geometry():
    for c, cap, first, kvf, q0 in [(0, 3, 0, 2, 0), (1, 3, 0, 4, 2), (2, 3, 0, 6, 4), (5, 3, 3, 6, 4), (5, 1, 5, 2, 0)]:
        f, pw = O.stream_window(CHUNK, c, cap)
        assert (f, pw.kv_frames, pw.q_frame0, pw.q_frames) == (first, kvf, q0, 2)
