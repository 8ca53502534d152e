"""CPU tests of the C-ABI library: it loads, exports what include/lcsa.h declares, the struct layout
matches the header, the host geometry (lcsa_csr_layout) agrees with the oracle's independently
written enumeration, and invalid problems are rejected before any device work."""
import ctypes
import glob
import os
import re
import subprocess

import numpy as np
import pytest

from block_sparse_causal_lcsa_amd import lcsa
from block_sparse_causal_lcsa_amd import workloads as W
from oracle import lcsa_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lcsa.h")
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    names = set()
    for path in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
        names.update(re.findall(r"\b(lcsa_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    lib = lcsa.load()
    names = declared_functions()
    assert set(names) == set(lcsa.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", lcsa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (lcsa_\w+)", out))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)
    assert lib.lcsa_version() == 100
    assert lib.lcsa_status_string(2) == b"LCSA_ERR_UNSUPPORTED"


def test_struct_layout_matches_header(tmp_path):
    src = tmp_path / "layout.c"
    fields = [f[0] for f in lcsa.LcsaProblem._fields_]
    body = "".join(f'printf("%zu ", offsetof(lcsa_problem, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "lcsa.h"\n'
                   f'int main(void){{ {body} printf("%zu %zu\\n", sizeof(lcsa_problem), sizeof(lcsa_strides)); return 0; }}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    want = [getattr(lcsa.LcsaProblem, f).offset for f in fields]
    assert got[:-2] == want
    assert got[-2:] == [ctypes.sizeof(lcsa.LcsaProblem), ctypes.sizeof(lcsa.LcsaStrides)]


def random_problems(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        Hb, Wb = int(rng.integers(1, 9)), int(rng.integers(1, 12))
        # every third problem has a ragged grid (partial last block row / column)
        dh, dw = (int(rng.integers(0, 8)), int(rng.integers(0, 8))) if len(out) % 3 == 2 else (0, 0)
        kvf = 2 * int(rng.integers(1, 5))
        qf = 2 * int(rng.integers(1, kvf // 2 + 1))
        q0 = 2 * int(rng.integers(0, (kvf - qf) // 2 + 1))
        mode = int(rng.integers(0, 5))   # none, block truncated / preserving, token truncated / preserving
        wb_h, wb_w = 2 * int(rng.integers(0, 5)) + 1, 2 * int(rng.integers(0, 5)) + 1
        if mode >= 3:                      # token windows: any positive size, in blocks' stead
            wb_h, wb_w = int(rng.integers(1, 40)) / 8, int(rng.integers(1, 40)) / 8
        topk = int(rng.integers(0, 6))
        rho = float(rng.choice([0.05, 0.136, 0.25, 1 / 3, 0.5, 0.77, 1.0]))
        out.append(W.Workload("r", 1, 2, 64, 8 * Hb - dh, 8 * Wb - dw, kvf, q0, qf, win_mode=mode,
                              win_h=int(8 * wb_h) if mode else 0, win_w=int(8 * wb_w) if mode else 0,
                              topk=topk, keep_ratio=rho))
    return out


@pytest.mark.parametrize("w", W.ALL + random_problems(40, 0), ids=lambda w: w.name)
def test_csr_layout_matches_oracle(w):
    nqb, nkb, nnz, rp = lcsa.lcsa_csr_layout(lcsa.problem(w))
    ref = O.csr_row_ptr(w)
    assert (nqb, nkb) == (w.nqb, w.nkb)
    assert nnz == ref[-1]
    assert np.array_equal(rp.astype(np.int64), ref)


BASE = W.CHUNK_768


@pytest.mark.parametrize("change,status", [
    (dict(head_dim=96), lcsa.LCSA_ERR_UNSUPPORTED),
    (dict(head_dim=0), lcsa.LCSA_ERR_UNSUPPORTED),
    (dict(grid_w=0), lcsa.LCSA_ERR_INVALID),
    (dict(blk_h=4), lcsa.LCSA_ERR_UNSUPPORTED),
    (dict(q_frame0=3, q_frames=2), lcsa.LCSA_ERR_UNSUPPORTED),
    (dict(kv_frames=7), lcsa.LCSA_ERR_UNSUPPORTED),
    (dict(q_frame0=6), lcsa.LCSA_ERR_INVALID),
    (dict(batch=0), lcsa.LCSA_ERR_INVALID),
    (dict(topk=-1), lcsa.LCSA_ERR_INVALID),
    (dict(keep_ratio=0.0), lcsa.LCSA_ERR_INVALID),
    (dict(keep_ratio=1.5), lcsa.LCSA_ERR_INVALID),
    (dict(keep_ratio=float("nan")), lcsa.LCSA_ERR_INVALID),
    (dict(win_mode=1, win_h=64, win_w=72), lcsa.LCSA_ERR_INVALID),
    (dict(win_mode=2, win_h=0, win_w=72), lcsa.LCSA_ERR_INVALID),
    (dict(win_mode=5, win_h=72, win_w=72), lcsa.LCSA_ERR_INVALID),
    (dict(win_mode=3, win_h=0, win_w=72), lcsa.LCSA_ERR_INVALID),
    # sums that would wrap in 32-bit arithmetic
    (dict(q_frame0=2**31 - 2, q_frames=2), lcsa.LCSA_ERR_INVALID),
    (dict(grid_h=2**31 - 1), lcsa.LCSA_ERR_UNSUPPORTED),
    (dict(grid_h=2**16, grid_w=2**16), lcsa.LCSA_ERR_UNSUPPORTED),
])
def test_invalid_problems_rejected_on_host(change, status):
    _check_rejected(BASE.replace(**change), status)


def test_nonpositive_scale_rejected_on_host():
    for scale in (0.0, -0.088, float("inf")):
        p = lcsa.problem(BASE)
        p.scale = scale
        _check_rejected(p, lcsa.LCSA_ERR_INVALID)


def _check_rejected(w_or_p, status):
    p = w_or_p if isinstance(w_or_p, lcsa.LcsaProblem) else lcsa.problem(w_or_p)
    lib = lcsa.load()
    assert lib.lcsa_csr_layout(ctypes.byref(p), None, None, None, None) == status
    assert lib.lcsa_last_error()
    # the device entry points validate first and return before touching HIP
    zs = lcsa.LcsaStrides(0, 0, 0)
    assert lib.lcsa_pool(ctypes.byref(p), None, zs, None, zs, None, None, None) == status
    assert lib.lcsa_score_select(ctypes.byref(p), None, None, None, None, None, None) == status
    assert lib.lcsa_attn_fwd(ctypes.byref(p), None, zs, None, zs, None, zs, None, None, None, zs, None, None) == status
    n = ctypes.c_size_t(0)
    assert lib.lcsa_attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == status
    assert lib.lcsa_attn_bwd(ctypes.byref(p), None, zs, None, zs, None, zs, None, zs, None, zs, None, None, None,
                             None, None, None, None, 0, None) == status


def test_bad_pointers_and_strides_rejected_on_host():
    lib = lcsa.load()
    p = lcsa.problem(BASE)
    d = BASE.head_dim
    good = lcsa.LcsaStrides(12 * 25344 * d, 25344 * d, d)
    buf = ctypes.c_void_p(1 << 20)   # never dereferenced: validation fails first
    mis = ctypes.c_void_p((1 << 20) + 8)
    zs = lcsa.LcsaStrides(0, 0, 0)
    assert lib.lcsa_pool(ctypes.byref(p), None, zs, None, zs, None, None, None) == lcsa.LCSA_ERR_INVALID
    assert lib.lcsa_pool(ctypes.byref(p), None, zs, mis, good, None, buf, None) == lcsa.LCSA_ERR_INVALID
    assert lib.lcsa_pool(ctypes.byref(p), None, zs, buf, lcsa.LcsaStrides(0, 0, d - 8), None, buf, None) \
        == lcsa.LCSA_ERR_INVALID
    assert lib.lcsa_pool(ctypes.byref(p), None, zs, buf, lcsa.LcsaStrides(0, 0, d + 4), None, buf, None) \
        == lcsa.LCSA_ERR_INVALID
    assert lib.lcsa_pool(ctypes.byref(p), None, zs, buf, good, None, None, None) == lcsa.LCSA_ERR_INVALID
    assert lib.lcsa_score_select(ctypes.byref(p), buf, buf, None, buf, None, None) == lcsa.LCSA_ERR_INVALID
    assert lib.lcsa_attn_fwd(ctypes.byref(p), buf, good, buf, good, buf, good, buf, buf, mis, good, None, None) \
        == lcsa.LCSA_ERR_INVALID
    assert b"aligned" in lib.lcsa_last_error()
    # output views whose rows overlap (two heads or two tokens on the same memory) are rejected:
    # zero head stride with 12 heads, and a head stride equal to the token stride
    nq = BASE.nq_tokens
    for os_ in (lcsa.LcsaStrides(12 * nq * d, 0, d), lcsa.LcsaStrides(12 * nq * d, d, d),
                lcsa.LcsaStrides(0, nq * d, d)):
        pp = lcsa.problem(BASE.replace(batch=2)) if os_.batch == 0 else p
        assert lib.lcsa_attn_fwd(ctypes.byref(pp), buf, good, buf, good, buf, good, buf, buf, buf, os_, None,
                                 None) == lcsa.LCSA_ERR_INVALID, (os_.batch, os_.head, os_.token)
        assert b"overlap" in lib.lcsa_last_error()
    # one query block whose candidates outnumber what LDS holds (a 200-frame cache at 1536x2688 with no
    # window: 25,200 candidate key blocks) is rejected; 40 frames at 768x1408 (1,320) are not
    huge = BASE.replace(grid_h=96, grid_w=168, kv_frames=200, q_frame0=198)
    ph = lcsa.problem(huge)
    assert lib.lcsa_score_select(ctypes.byref(ph), buf, buf, buf, buf, None, None) == lcsa.LCSA_ERR_UNSUPPORTED
    assert b"exceed" in lib.lcsa_last_error()


def test_backward_rejections_on_host():
    lib = lcsa.load()
    p = lcsa.problem(BASE)
    d = BASE.head_dim
    hw = BASE.grid_h * BASE.grid_w
    qs = lcsa.LcsaStrides(12 * 2 * hw * d, 2 * hw * d, d)
    ks = lcsa.LcsaStrides(12 * 6 * hw * d, 6 * hw * d, d)
    buf = ctypes.c_void_p(1 << 20)   # never dereferenced: validation fails first
    n = ctypes.c_size_t(0)
    assert lib.lcsa_attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == lcsa.LCSA_OK
    nqb, nkb, nnz, _ = lcsa.lcsa_csr_layout(p)
    # delta and lse2 [B*Hh*Nq] fp32, col_ptr [B*Hh*(nkb+1)] and row_of [B*Hh*nnz] int32, each 256-byte rounded
    up = lambda x: (x + 255) // 256 * 256
    assert n.value == 2 * up(12 * 2 * hw * 4) + up(12 * (nkb + 1) * 4) + up(12 * nnz * 4)
    assert lib.lcsa_attn_bwd_workspace_size(ctypes.byref(p), None) == lcsa.LCSA_ERR_INVALID

    def call(prob=p, lse=buf, ws=buf, wsb=n.value, dq=buf):
        return lib.lcsa_attn_bwd(ctypes.byref(prob), buf, qs, buf, ks, buf, ks, buf, qs, buf, qs, lse, buf, buf,
                                 dq, buf, buf, ws, wsb, None)

    assert call(lse=None) == lcsa.LCSA_ERR_INVALID
    assert call(ws=None) == lcsa.LCSA_ERR_INVALID
    assert call(wsb=n.value - 1) == lcsa.LCSA_ERR_INVALID
    assert b"workspace" in lib.lcsa_last_error()
    assert call(dq=ctypes.c_void_p((1 << 20) + 8)) == lcsa.LCSA_ERR_INVALID
    assert call(ws=ctypes.c_void_p((1 << 20) + 128)) == lcsa.LCSA_ERR_INVALID
    pf = lcsa.problem(BASE.replace(dtype="f32"))
    assert call(prob=pf) == lcsa.LCSA_ERR_UNSUPPORTED
    assert b"bf16" in lib.lcsa_last_error()


def test_noalloc_backward_rejects_a_problem_beyond_its_scratch_on_host():
    # a 26-frame clip at 1536x2688 needs more workspace than the static scratch array holds: rejected
    # during validation, before any HIP call
    lib = lcsa.load()
    big = W.UHD_TRUNC.replace(kv_frames=26, q_frame0=0, q_frames=26)
    p = lcsa.problem(big)
    n = ctypes.c_size_t(0)
    assert lib.lcsa_attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)) == lcsa.LCSA_OK
    assert n.value > lcsa.NOALLOC_SCRATCH_BYTES
    buf = ctypes.c_void_p(1 << 20)   # never dereferenced
    st = lcsa.LcsaStrides(big.heads * big.nq_tokens * big.head_dim, big.nq_tokens * big.head_dim, big.head_dim)
    r = lib.lcsa_attn_bwd_noalloc(ctypes.byref(p), buf, st, buf, st, buf, st, buf, st, buf, st, buf, buf, buf,
                                  buf, buf, buf, None)
    assert r == lcsa.LCSA_ERR_UNSUPPORTED
    assert b"static scratch" in lib.lcsa_last_error()
    # and a NULL gradient is still rejected as invalid
    r = lib.lcsa_attn_bwd_noalloc(ctypes.byref(p), buf, st, buf, st, buf, st, buf, st, buf, st, buf, buf, buf,
                                  None, buf, buf, None)
    assert r == lcsa.LCSA_ERR_INVALID


def test_stream_struct_layout_matches_header(tmp_path):
    src = tmp_path / "slayout.c"
    fields = [f[0] for f in lcsa.LcsaStream._fields_]
    body = "".join(f'printf("%zu ", offsetof(lcsa_stream, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "lcsa.h"\n'
                   f'int main(void){{ {body} printf("%zu\\n", sizeof(lcsa_stream)); return 0; }}\n')
    exe = tmp_path / "slayout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    assert got[:-1] == [getattr(lcsa.LcsaStream, f).offset for f in fields]
    assert got[-1] == ctypes.sizeof(lcsa.LcsaStream)


def test_stream_state_on_host():
    lib = lcsa.load()
    chunk = BASE.replace(kv_frames=2, q_frame0=0, q_frames=2)
    p = lcsa.problem(chunk)
    n = ctypes.c_size_t(0)
    assert lib.lcsa_stream_state_size(ctypes.byref(p), 3, 7, ctypes.byref(n)) == lcsa.LCSA_OK
    # K and V rings of 7 temporal-block slots (bf16) + two pooled-K buffers of 3 blocks' means (fp32)
    hw, d, Hh = BASE.grid_h * BASE.grid_w, BASE.head_dim, BASE.heads
    blk = 2 * hw * d * 2                   # bytes of one temporal block of one head
    ring = Hh * 7 * blk
    kbar = Hh * 3 * (hw // 64) * d * 4
    up = lambda x: (x + 255) // 256 * 256
    assert n.value == 2 * up(ring) + 2 * up(kbar)
    assert lib.lcsa_stream_state_size(ctypes.byref(p), 0, 7, ctypes.byref(n)) == lcsa.LCSA_ERR_INVALID
    assert lib.lcsa_stream_state_size(ctypes.byref(p), 3, 4, ctypes.byref(n)) == lcsa.LCSA_ERR_INVALID
    assert lib.lcsa_stream_state_size(ctypes.byref(p), 1, 1, ctypes.byref(n)) == lcsa.LCSA_OK
    p4 = lcsa.problem(BASE.replace(kv_frames=4, q_frame0=0, q_frames=4))
    assert lib.lcsa_stream_state_size(ctypes.byref(p4), 3, 7, ctypes.byref(n)) == lcsa.LCSA_ERR_UNSUPPORTED
    st = lcsa.LcsaStream()
    mem = ctypes.c_void_p(1 << 20)   # never dereferenced: no device work on these paths
    assert lib.lcsa_stream_init(ctypes.byref(st), ctypes.byref(p), 3, 7, mem, 1024) == lcsa.LCSA_ERR_INVALID
    assert b"needed" in lib.lcsa_last_error()
    assert lib.lcsa_stream_init(ctypes.byref(st), ctypes.byref(p), 3, 7, ctypes.c_void_p((1 << 20) + 64),
                                1 << 40) == lcsa.LCSA_ERR_INVALID
    assert lib.lcsa_stream_init(ctypes.byref(st), ctypes.byref(p), 3, 7, mem, 1 << 40) == lcsa.LCSA_OK
    assert (st.held, st.pushed, st.wpos, st.cache_tblocks, st.ring_tblocks) == (0, 0, 0, 3, 7)
    wp = lcsa.LcsaProblem()
    assert lib.lcsa_stream_window(ctypes.byref(st), ctypes.byref(wp), None, None, None, None, None) \
        == lcsa.LCSA_ERR_INVALID
    zs = lcsa.LcsaStrides(0, 0, 0)
    assert lib.lcsa_stream_push(ctypes.byref(st), None, zs, None, zs, None) == lcsa.LCSA_ERR_INVALID
    assert (st.held, st.pushed, st.wpos) == (0, 0, 0)
    # reserve below the end of the ring: no device work, the slot at wpos
    ks = lcsa.LcsaStrides()
    k = ctypes.c_void_p()
    st.wpos = 4
    st.held = 3
    st.pushed = 9
    assert lib.lcsa_stream_reserve(ctypes.byref(st), ctypes.byref(k), ctypes.byref(ks), None, None, None) \
        == lcsa.LCSA_OK
    assert k.value == (1 << 20) + 4 * blk and (ks.batch, ks.head, ks.token) == (Hh * 7 * 2 * hw * d, 7 * 2 * hw * d, d)
    # window geometry from the host bookkeeping alone (no device work)
    for pushed, held, wpos, kvf in [(1, 1, 1, 2), (2, 2, 2, 4), (3, 3, 3, 6), (9, 3, 4, 6), (8, 3, 7, 6)]:
        st.pushed, st.held, st.wpos = pushed, held, wpos
        k, v, kb = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
        vs = lcsa.LcsaStrides()
        assert lib.lcsa_stream_window(ctypes.byref(st), ctypes.byref(wp), ctypes.byref(k), ctypes.byref(ks),
                                      ctypes.byref(v), ctypes.byref(vs), ctypes.byref(kb)) == lcsa.LCSA_OK
        assert (wp.kv_frames, wp.q_frame0, wp.q_frames) == (kvf, kvf - 2, 2)
        assert k.value == (1 << 20) + (wpos - held) * blk
        assert v.value == (1 << 20) + up(ring) + (wpos - held) * blk
        assert kb.value == (1 << 20) + 2 * up(ring) + (0 if pushed % 2 else up(kbar))
    st.wpos = 2   # just after a compacting reserve: no window until the push
    assert lib.lcsa_stream_window(ctypes.byref(st), ctypes.byref(wp), None, None, None, None, None) \
        == lcsa.LCSA_ERR_INVALID
    assert b"compacted" in lib.lcsa_last_error()
    st.wpos = 1   # fewer slots than that: rejected as an uninitialised state
    assert lib.lcsa_stream_window(ctypes.byref(st), ctypes.byref(wp), None, None, None, None, None) \
        == lcsa.LCSA_ERR_INVALID
    assert b"not initialised" in lib.lcsa_last_error()


def test_rope_rejections_on_host():
    lib = lcsa.load()
    chunk = BASE.replace(kv_frames=2, q_frame0=0, q_frames=2)
    p = lcsa.problem(chunk)
    d = BASE.head_dim
    hw = BASE.grid_h * BASE.grid_w
    buf = ctypes.c_void_p(1 << 20)   # never dereferenced: validation fails first
    st = lcsa.LcsaStrides(12 * 2 * hw * d, 2 * hw * d, d)
    row = 3 * 12 * d

    def call(rope, frames=2, qkv=buf, tok=row, prob=p):
        r = ctypes.byref(rope) if rope is not None else None
        return lib.lcsa_rope_qkv(ctypes.byref(prob), r, qkv, 2 * hw * row, tok, 0, frames, buf, st, buf, st, buf, st,
                                 None)

    assert call(None) == lcsa.LCSA_ERR_INVALID
    assert call(lcsa.LcsaRope(44, 42, 40, 10000.0)) == lcsa.LCSA_ERR_INVALID       # sum != head_dim
    assert call(lcsa.LcsaRope(43, 43, 42, 10000.0)) == lcsa.LCSA_ERR_INVALID       # odd dims
    assert call(lcsa.LcsaRope(44, 42, 42, 1.0)) == lcsa.LCSA_ERR_INVALID           # theta
    assert call(lcsa.LcsaRope(44, 42, 42, 10000.0), frames=3) == lcsa.LCSA_ERR_INVALID
    assert call(lcsa.LcsaRope(44, 42, 42, 10000.0), tok=row - 8) == lcsa.LCSA_ERR_INVALID
    assert call(lcsa.LcsaRope(44, 42, 42, 10000.0), qkv=ctypes.c_void_p((1 << 20) + 4)) == lcsa.LCSA_ERR_INVALID
    # an output view with every head on the same rows
    r = lcsa.LcsaRope(44, 42, 42, 10000.0)
    assert lib.lcsa_rope_qkv(ctypes.byref(p), ctypes.byref(r), buf, 2 * hw * row, row, 0, 2, buf, st, buf,
                             lcsa.LcsaStrides(12 * 2 * hw * d, 0, d), buf, st, None) == lcsa.LCSA_ERR_INVALID
    assert b"overlap" in lib.lcsa_last_error()
    pf = lcsa.problem(chunk.replace(dtype="f32"))
    assert call(lcsa.LcsaRope(44, 42, 42, 10000.0), prob=pf) == lcsa.LCSA_ERR_UNSUPPORTED


def test_rope_struct_layout_matches_header(tmp_path):
    src = tmp_path / "rlayout.c"
    fields = [f[0] for f in lcsa.LcsaRope._fields_]
    body = "".join(f'printf("%zu ", offsetof(lcsa_rope, {f}));' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "lcsa.h"\n'
                   f'int main(void){{ {body} printf("%zu\\n", sizeof(lcsa_rope)); return 0; }}\n')
    exe = tmp_path / "rlayout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    assert got[:-1] == [getattr(lcsa.LcsaRope, f).offset for f in fields]
    assert got[-1] == ctypes.sizeof(lcsa.LcsaRope)


def test_binding_rejects_host_tensors():
    """Host (CPU) tensors never reach the library: each call raises before any device work."""
    import torch
    w = W.Workload("host_check", 1, 2, 64, 16, 16, 4, 2, 2)
    p = lcsa.problem(w)
    nq, nk = 2 * 16 * 16, 4 * 16 * 16
    q = torch.zeros((1, 2, nq, 64), dtype=torch.bfloat16)
    k = torch.zeros((1, 2, nk, 64), dtype=torch.bfloat16)
    v = torch.zeros_like(k)
    nqb, nkb, nnz, rp = lcsa.lcsa_csr_layout(p)
    row_ptr = torch.from_numpy(rp)
    col = torch.zeros((1, 2, nnz), dtype=torch.int32)
    with pytest.raises(ValueError, match="device tensor"):
        lcsa.lcsa_pool(p, q, k)
    with pytest.raises(ValueError, match="device tensor"):
        lcsa.lcsa_score_select(p, torch.zeros((1, 2, nqb, 64)), torch.zeros((1, 2, nkb, 64)), row_ptr)
    with pytest.raises(ValueError, match="device tensor"):
        lcsa.lcsa_attn_fwd(p, q, k, v, row_ptr, col)
    with pytest.raises(ValueError, match="device tensor"):
        lcsa.lcsa_attn_bwd(p, q, k, v, q, q, torch.zeros((1, 2, nq)), row_ptr, col)
    with pytest.raises(ValueError, match="device tensor"):
        lcsa.lcsa_rope_qkv(p, lcsa.LcsaRope(22, 20, 22, 10000.0), torch.zeros((1, nq, 3 * 2 * 64), dtype=torch.bfloat16), 2)


def test_mfma_probe_rejects_bad_arguments_on_host():
    lib = lcsa.load()
    flop = ctypes.c_double(-1.0)
    sink = ctypes.c_void_p(16)
    for wg, it in ((0, 10), (1 << 21, 10), (4, 0), (4, 1 << 25)):
        assert lib.lcsa_mfma_probe(wg, it, sink, ctypes.byref(flop), None) == lcsa.LCSA_ERR_INVALID
    assert lib.lcsa_mfma_probe(4, 10, None, ctypes.byref(flop), None) == lcsa.LCSA_ERR_INVALID
    assert lib.lcsa_mfma_probe(4, 10, ctypes.c_void_p(18), ctypes.byref(flop), None) == lcsa.LCSA_ERR_INVALID
    assert flop.value == -1.0  # nothing written before validation passes
