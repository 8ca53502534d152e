"""GPU parity on seeded random problems: every stage of the forward (pooling, scores, selection,
attention) and, for bf16 problems, the backward, against the fp64 oracle at the bars of parity.py
and test_gpu_backward.py.

The problems mix what the fixed cases cover one at a time: grids that are and are not multiples of
8, batch 1-2, 1-3 heads, head_dim 64 and 128, bf16 and fp32 I/O, query frames anywhere inside the
key frames, every window rule (none, block truncated / preserving with odd block widths, token
truncated / preserving with any positive width, also wider than the grid), and Top-K by count or by
keep ratio. Sizes stay small so the oracle checks every row.
"""
import numpy as np
import pytest

from block_sparse_causal_lcsa_amd import workloads as W
from oracle import lcsa_oracle as O

from parity import full_check
from test_gpu_backward import check_unkept_zero, compare, report, run

pytestmark = pytest.mark.gpu


def random_problems(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for idx in range(n):
        Hb, Wb = int(rng.integers(1, 6)), int(rng.integers(1, 7))
        ragged = idx % 2 == 1
        dh, dw = (int(rng.integers(0, 8)), int(rng.integers(0, 8))) if ragged else (0, 0)
        H, Wd = max(1, 8 * Hb - dh), max(1, 8 * Wb - dw)
        kvf = 2 * int(rng.integers(1, 4))
        qf = 2 * int(rng.integers(1, kvf // 2 + 1))
        q0 = 2 * int(rng.integers(0, (kvf - qf) // 2 + 1))
        mode = int(rng.integers(0, 5))
        if mode in (1, 2):
            win_h, win_w = 8 * (2 * int(rng.integers(0, 4)) + 1), 8 * (2 * int(rng.integers(0, 4)) + 1)
        elif mode in (3, 4):
            win_h, win_w = int(rng.integers(1, 2 * H + 2)), int(rng.integers(1, 2 * Wd + 2))
        else:
            win_h = win_w = 0
        topk = int(rng.choice([0, 0, 1, 2, 5]))
        rho = float(rng.choice([0.05, 0.2, 0.5, 1.0]))
        dtype = "f32" if idx % 5 == 4 else "bf16"
        d = int(rng.choice([64, 128]))
        batch, heads = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        name = (f"rand{idx}_{batch}x{heads}_d{d}_{dtype}_{H}x{Wd}_f{q0}+{qf}of{kvf}_w{mode}"
                f"-{win_h}x{win_w}_k{topk or rho}")
        out.append(W.Workload(name, batch, heads, d, H, Wd, kvf, q0, qf, dtype=dtype, win_mode=mode,
                              win_h=win_h, win_w=win_w, topk=topk, keep_ratio=rho))
    return out


PROBLEMS = random_problems(16, 2024) + [w.replace(name=w.name.replace("rand", "rnd")) for w in random_problems(24, 99)]


@pytest.mark.parametrize("w", PROBLEMS, ids=lambda w: w.name)
def test_random_forward(w):
    stats = full_check(w, seed=7)
    print(f"PARITY {w.name} {stats}", flush=True)


@pytest.mark.parametrize("w", [w for w in PROBLEMS if w.dtype == "bf16"], ids=lambda w: w.name)
def test_random_backward(w):
    r = run(w, 3)
    q, k, v = r["x64"]
    dQ, dK, dV = O.attend_bwd(w, q, k, v, r["row_ptr"], r["col"], r["g64"])
    # rows that see no kept key (token windows) have zero gradients on both sides; compare the rest
    # of every tensor, and the whole tensor when nothing is zero
    stats = {}
    for n, ref in (("dq", dQ), ("dk", dK), ("dv", dV)):
        m = np.ones(ref.shape[:3], dtype=bool)
        if np.any(np.abs(ref).sum(axis=-1) > 0):
            stats[n] = compare(n, r[n], ref, m)
        else:
            assert not np.any(r[n]), f"{n}: oracle gradient is zero, GPU's is not"
    stats["unkept_key_blocks"] = check_unkept_zero(w, r)
    report(w.name, stats)


def random_streams(n, seed):
    """(sequence workload, cache blocks, ring blocks, chunks pushed in place) per random stream."""
    rng = np.random.default_rng(seed)
    out = []
    for idx in range(n):
        H, Wd = int(rng.integers(3, 33)), int(rng.integers(3, 41))
        nchunks = int(rng.integers(2, 9))
        cache = int(rng.integers(1, 5))
        ring = 0 if idx % 2 == 0 else 2 * cache - 1 + int(rng.integers(0, 4))
        mode = int(rng.integers(0, 5))
        if mode in (1, 2):
            win_h, win_w = 8 * (2 * int(rng.integers(0, 3)) + 1), 8 * (2 * int(rng.integers(0, 3)) + 1)
        elif mode in (3, 4):
            win_h, win_w = int(rng.integers(1, 2 * H + 2)), int(rng.integers(1, 2 * Wd + 2))
        else:
            win_h = win_w = 0
        topk = int(rng.choice([0, 0, 1, 3]))
        rho = float(rng.choice([0.1, 0.3, 0.6, 1.0]))
        dtype = "f32" if idx % 4 == 3 else "bf16"
        d = int(rng.choice([64, 128]))
        batch, heads = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        in_place = tuple(int(c) for c in rng.choice(nchunks, size=min(2, nchunks), replace=False))
        name = (f"rstream{idx}_{batch}x{heads}_d{d}_{dtype}_{H}x{Wd}_c{cache}r{ring}_n{nchunks}_w{mode}"
                f"-{win_h}x{win_w}_k{topk or rho}")
        seq = W.Workload(name, batch, heads, d, H, Wd, 2 * nchunks, 0, 2 * nchunks, dtype=dtype, win_mode=mode,
                         win_h=win_h, win_w=win_w, topk=topk, keep_ratio=rho)
        out.append((seq, cache, ring, in_place))
    return out


STREAMS = random_streams(8, 77)


@pytest.mark.parametrize("case", STREAMS, ids=lambda c: c[0].name)
def test_random_stream(case):
    from test_gpu_stream import run_stream
    seq, cache, ring, in_place = case
    nchunks = seq.kv_frames // 2
    run_stream(seq, cache, seed=5, oracle_chunks=(0, nchunks - 1), ring=ring, in_place=in_place)
