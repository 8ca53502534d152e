"""Thin Python binding of liblcsa.so (ctypes). Argument marshalling only: every step of the LCSA
forward runs in the library's HIP kernels; torch provides device memory and the stream.

The functions carry the C names: lcsa_csr_layout, lcsa_pool, lcsa_score_select, lcsa_attn_fwd,
lcsa_attn_bwd_workspace_size, lcsa_attn_bwd. `forward` chains the three forward device calls on the
current stream.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
# LCSA_LIBRARY may name another build of the same library (the host-sanitized one that the CPU
# tests load); by default the in-tree liblcsa.so is loaded.
LIB_PATH = os.environ.get("LCSA_LIBRARY") or os.path.join(_PKG, "liblcsa.so")

LCSA_OK, LCSA_ERR_INVALID, LCSA_ERR_UNSUPPORTED, LCSA_ERR_HIP = 0, 1, 2, 3
LCSA_BF16, LCSA_F32 = 0, 1

EXPORTS = ("lcsa_csr_layout", "lcsa_pool", "lcsa_score_select", "lcsa_attn_fwd",
           "lcsa_attn_bwd_workspace_size", "lcsa_attn_bwd", "lcsa_attn_bwd_noalloc",
           "lcsa_stream_state_size", "lcsa_stream_init", "lcsa_stream_reserve", "lcsa_stream_push",
           "lcsa_stream_window", "lcsa_rope_qkv", "lcsa_mfma_probe",
           "lcsa_status_string", "lcsa_last_error", "lcsa_version")


class LcsaProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "heads", "head_dim", "grid_h", "grid_w", "kv_frames", "q_frame0", "q_frames",
        "blk_t", "blk_h", "blk_w", "win_mode", "win_h", "win_w", "topk")] + [
        ("keep_ratio", ctypes.c_double), ("scale", ctypes.c_float), ("dtype", ctypes.c_int32)]


class LcsaStrides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("token", ctypes.c_int64)]


class LcsaStream(ctypes.Structure):
    _fields_ = [("chunk", LcsaProblem), ("cache_tblocks", ctypes.c_int32), ("ring_tblocks", ctypes.c_int32),
                ("held", ctypes.c_int32), ("wpos", ctypes.c_int32), ("pushed", ctypes.c_int64),
                ("mem", ctypes.c_void_p), ("mem_bytes", ctypes.c_size_t)]


class LcsaRope(ctypes.Structure):
    _fields_ = [("dim_t", ctypes.c_int32), ("dim_h", ctypes.c_int32), ("dim_w", ctypes.c_int32),
                ("theta", ctypes.c_float)]


class LcsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


_lib = None


def load():
    """Loads liblcsa.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_sparse_causal_lcsa_amd.build` (or __graft_entry__.build())")
    # The library must run on the same HIP runtime instance that owns the caller's device memory
    # and streams. torch ships its own libamdhip64; importing torch first makes the dynamic loader
    # bind liblcsa.so to that instance (same soname) instead of mapping a second runtime.
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P, S, vp = ctypes.POINTER(LcsaProblem), LcsaStrides, ctypes.c_void_p
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.lcsa_csr_layout.argtypes = [P, i32p, i32p, i32p, i32p]
    lib.lcsa_pool.argtypes = [P, vp, S, vp, S, vp, vp, vp]
    lib.lcsa_score_select.argtypes = [P, vp, vp, vp, vp, vp, vp]
    lib.lcsa_attn_fwd.argtypes = [P, vp, S, vp, S, vp, S, vp, vp, vp, S, vp, vp]
    lib.lcsa_attn_bwd_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.lcsa_attn_bwd.argtypes = [P, vp, S, vp, S, vp, S, vp, S, vp, S, vp, vp, vp, vp, vp, vp, vp,
                                  ctypes.c_size_t, vp]
    lib.lcsa_attn_bwd_noalloc.argtypes = [P, vp, S, vp, S, vp, S, vp, S, vp, S, vp, vp, vp, vp, vp, vp, vp]
    lib.lcsa_rope_qkv.argtypes = [P, ctypes.POINTER(LcsaRope), vp, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_int32, vp, S, vp, S, vp, S, vp]
    SP = ctypes.POINTER(LcsaStream)
    lib.lcsa_stream_state_size.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)]
    lib.lcsa_stream_init.argtypes = [SP, P, ctypes.c_int32, ctypes.c_int32, vp, ctypes.c_size_t]
    lib.lcsa_stream_reserve.argtypes = [SP, ctypes.POINTER(vp), ctypes.POINTER(S), ctypes.POINTER(vp),
                                        ctypes.POINTER(S), vp]
    lib.lcsa_stream_push.argtypes = [SP, vp, S, vp, S, vp]
    lib.lcsa_stream_window.argtypes = [SP, P, ctypes.POINTER(vp), ctypes.POINTER(S), ctypes.POINTER(vp),
                                       ctypes.POINTER(S), ctypes.POINTER(vp)]
    lib.lcsa_mfma_probe.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, ctypes.POINTER(ctypes.c_double), vp]
    for f in ("lcsa_csr_layout", "lcsa_pool", "lcsa_score_select", "lcsa_attn_fwd",
              "lcsa_attn_bwd_workspace_size", "lcsa_attn_bwd", "lcsa_attn_bwd_noalloc", "lcsa_stream_state_size", "lcsa_stream_init",
              "lcsa_stream_reserve", "lcsa_stream_push", "lcsa_stream_window", "lcsa_rope_qkv", "lcsa_mfma_probe"):
        getattr(lib, f).restype = ctypes.c_int
    lib.lcsa_status_string.argtypes = [ctypes.c_int]
    lib.lcsa_status_string.restype = ctypes.c_char_p
    lib.lcsa_last_error.argtypes = []
    lib.lcsa_last_error.restype = ctypes.c_char_p
    lib.lcsa_version.restype = ctypes.c_int32
    _lib = lib
    return lib


def _status_name(s: int) -> str:
    return {0: "LCSA_OK", 1: "LCSA_ERR_INVALID", 2: "LCSA_ERR_UNSUPPORTED", 3: "LCSA_ERR_HIP"}.get(s, str(s))


def _check(status: int):
    if status != LCSA_OK:
        raise LcsaError(status, load().lcsa_last_error().decode())


def problem(w) -> LcsaProblem:
    """LcsaProblem from any object with the Workload attributes."""
    return LcsaProblem(batch=w.batch, heads=w.heads, head_dim=w.head_dim, grid_h=w.grid_h, grid_w=w.grid_w,
                       kv_frames=w.kv_frames, q_frame0=w.q_frame0, q_frames=w.q_frames, blk_t=w.blk_t,
                       blk_h=w.blk_h, blk_w=w.blk_w, win_mode=w.win_mode, win_h=w.win_h, win_w=w.win_w,
                       topk=w.topk, keep_ratio=w.keep_ratio, scale=w.scale,
                       dtype=LCSA_F32 if w.dtype == "f32" else LCSA_BF16)


def lcsa_csr_layout(p: LcsaProblem):
    """Returns (nqb, nkb, nnz_per_head, row_ptr int32 numpy [nqb+1]); host only."""
    lib = load()
    nqb, nkb, nnz = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib.lcsa_csr_layout(ctypes.byref(p), ctypes.byref(nqb), ctypes.byref(nkb), ctypes.byref(nnz), None))
    rp = np.zeros(nqb.value + 1, dtype=np.int32)
    _check(lib.lcsa_csr_layout(ctypes.byref(p), None, None, None,
                               rp.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))))
    return nqb.value, nkb.value, nnz.value, rp


# ------------------------------------------------------------------------------- device calls
def _torch():
    import torch
    return torch


def _strides(t) -> LcsaStrides:
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("token tensors must be [batch, heads, tokens, head_dim] with unit head_dim stride")
    return LcsaStrides(t.stride(0), t.stride(1), t.stride(2))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype(p: LcsaProblem):
    torch = _torch()
    return torch.float32 if p.dtype == LCSA_F32 else torch.bfloat16


def _on_device(name, t):
    """Every pointer handed to the library must be device memory of the current device."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, the current device is cuda:{torch.cuda.current_device()}")


def _check_buffer(name, t, dtype, numel):
    """A contiguous device tensor of `dtype` with exactly `numel` elements."""
    _on_device(name, t)
    if t.dtype != dtype or not t.is_contiguous() or t.numel() != numel:
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor of {numel} elements")


_COUNTS = {}


def _block_counts(p: LcsaProblem):
    """(nqb, nkb, nnz_per_head) of a problem, cached by its bytes (host only)."""
    key = bytes(p)
    v = _COUNTS.get(key)
    if v is None:
        if len(_COUNTS) > 1024:
            _COUNTS.clear()
        v = _COUNTS[key] = lcsa_csr_layout(p)[:3]
    return v


def _check_selection(p, row_ptr, col_idx, nqb, nnz):
    torch = _torch()
    _check_buffer("row_ptr", row_ptr, torch.int32, nqb + 1)
    if col_idx is not None:
        _check_buffer("col_idx", col_idx, torch.int32, p.batch * p.heads * nnz)


def _check_token_tensor(name, t, p, ntok):
    torch = _torch()
    _on_device(name, t)
    if t.dtype != _dtype(p):
        raise ValueError(f"{name} has dtype {t.dtype}, problem expects {_dtype(p)}")
    if tuple(t.shape) != (p.batch, p.heads, ntok, p.head_dim):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(p.batch, p.heads, ntok, p.head_dim)}")
    return torch


def lcsa_pool(p: LcsaProblem, q, k, q_pooled=None, k_pooled=None, stream=None):
    """Block means of q and k (either may be None) -> (q_pooled, k_pooled) fp32 device tensors."""
    torch = _torch()
    nqb, nkb, _ = _block_counts(p)
    hw = p.grid_h * p.grid_w
    if q is not None:
        _check_token_tensor("q", q, p, p.q_frames * hw)
        if q_pooled is None:
            q_pooled = torch.empty((p.batch, p.heads, nqb, p.head_dim), dtype=torch.float32, device=q.device)
        _check_buffer("q_pooled", q_pooled, torch.float32, p.batch * p.heads * nqb * p.head_dim)
    if k is not None:
        _check_token_tensor("k", k, p, p.kv_frames * hw)
        if k_pooled is None:
            k_pooled = torch.empty((p.batch, p.heads, nkb, p.head_dim), dtype=torch.float32, device=k.device)
        _check_buffer("k_pooled", k_pooled, torch.float32, p.batch * p.heads * nkb * p.head_dim)
    zs = LcsaStrides(0, 0, 0)
    _check(load().lcsa_pool(ctypes.byref(p), _ptr(q), _strides(q) if q is not None else zs, _ptr(k),
                            _strides(k) if k is not None else zs, _ptr(q_pooled if q is not None else None),
                            _ptr(k_pooled if k is not None else None), _stream(stream)))
    return q_pooled, k_pooled


def lcsa_score_select(p: LcsaProblem, q_pooled, k_pooled, row_ptr, col_idx=None, scores_dbg=None, stream=None):
    """Per-row Top-K key blocks -> col_idx int32 [B, Hh, nnz_per_head] (row_ptr: device int32)."""
    torch = _torch()
    nqb, nkb, nnz = _block_counts(p)
    for name, t, n in (("q_pooled", q_pooled, nqb), ("k_pooled", k_pooled, nkb)):
        _on_device(name, t)
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (p.batch, p.heads, n, p.head_dim):
            raise ValueError(f"{name} must be contiguous fp32 [{p.batch}, {p.heads}, {n}, {p.head_dim}]")
    if col_idx is None:
        col_idx = torch.empty((p.batch, p.heads, nnz), dtype=torch.int32, device=q_pooled.device)
    _check_selection(p, row_ptr, col_idx, nqb, nnz)
    if scores_dbg is not None:
        _check_buffer("scores_dbg", scores_dbg, torch.float64, p.batch * p.heads * nqb * nkb)
    _check(load().lcsa_score_select(ctypes.byref(p), _ptr(q_pooled), _ptr(k_pooled), _ptr(row_ptr), _ptr(col_idx),
                                    _ptr(scores_dbg), _stream(stream)))
    return col_idx


def lcsa_attn_fwd(p: LcsaProblem, q, k, v, row_ptr, col_idx, o=None, lse=None, want_lse=True, stream=None):
    """Exact attention over the kept blocks -> (o, lse)."""
    torch = _torch()
    hw = p.grid_h * p.grid_w
    _check_token_tensor("q", q, p, p.q_frames * hw)
    _check_token_tensor("k", k, p, p.kv_frames * hw)
    _check_token_tensor("v", v, p, p.kv_frames * hw)
    if o is None:
        o = torch.empty_like(q)
    _check_token_tensor("o", o, p, p.q_frames * hw)
    if lse is None and want_lse:
        lse = torch.empty((p.batch, p.heads, p.q_frames * hw), dtype=torch.float32, device=q.device)
    if lse is not None:
        _check_buffer("lse", lse, torch.float32, p.batch * p.heads * p.q_frames * hw)
    nqb, _, nnz = _block_counts(p)
    _check_selection(p, row_ptr, col_idx, nqb, nnz)
    _check(load().lcsa_attn_fwd(ctypes.byref(p), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                                _ptr(row_ptr), _ptr(col_idx), _ptr(o), _strides(o), _ptr(lse), _stream(stream)))
    return o, lse


def lcsa_attn_bwd_workspace_size(p: LcsaProblem) -> int:
    """Bytes of device workspace lcsa_attn_bwd needs for this problem (host only)."""
    n = ctypes.c_size_t()
    _check(load().lcsa_attn_bwd_workspace_size(ctypes.byref(p), ctypes.byref(n)))
    return n.value


def lcsa_attn_bwd(p: LcsaProblem, q, k, v, o, d_o, lse, row_ptr, col_idx, dq=None, dk=None, dv=None,
                  workspace=None, stream=None):
    """Gradients of lcsa_attn_fwd for a fixed selection -> (dq, dk, dv) fp32 device tensors."""
    torch = _torch()
    hw = p.grid_h * p.grid_w
    nq, nk = p.q_frames * hw, p.kv_frames * hw
    for name, t, n in (("q", q, nq), ("k", k, nk), ("v", v, nk), ("o", o, nq), ("d_o", d_o, nq)):
        _check_token_tensor(name, t, p, n)
    if lse is None:
        raise ValueError("lse (the forward's output) is required")
    _check_buffer("lse", lse, torch.float32, p.batch * p.heads * nq)
    nqb, _, nnz = _block_counts(p)
    _check_selection(p, row_ptr, col_idx, nqb, nnz)
    grads = []
    for name, t, n in (("dq", dq, nq), ("dk", dk, nk), ("dv", dv, nk)):
        if t is None:
            t = torch.empty((p.batch, p.heads, n, p.head_dim), dtype=torch.float32, device=q.device)
        _on_device(name, t)
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (p.batch, p.heads, n, p.head_dim):
            raise ValueError(f"{name} must be contiguous fp32 [{p.batch}, {p.heads}, {n}, {p.head_dim}]")
        grads.append(t)
    need = lcsa_attn_bwd_workspace_size(p)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _on_device("workspace", workspace)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    _check(load().lcsa_attn_bwd(ctypes.byref(p), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v), _strides(v),
                                _ptr(o), _strides(o), _ptr(d_o), _strides(d_o), _ptr(lse), _ptr(row_ptr),
                                _ptr(col_idx), _ptr(grads[0]), _ptr(grads[1]), _ptr(grads[2]), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)))
    return tuple(grads)


NOALLOC_SCRATCH_BYTES = 16 << 20   # LCSA_NOALLOC_SCRATCH_BYTES in lcsa.h


def lcsa_attn_bwd_noalloc(p: LcsaProblem, q, k, v, o, d_o, lse, row_ptr, col_idx, dq, dk, dv, stream=None):
    """lcsa_attn_bwd on the library's static per-GPU scratch array: no workspace argument and no
    allocation anywhere in the call (dq, dk, dv are the caller's)."""
    hw = p.grid_h * p.grid_w
    nq, nk = p.q_frames * hw, p.kv_frames * hw
    for name, t, n in (("q", q, nq), ("k", k, nk), ("v", v, nk), ("o", o, nq), ("d_o", d_o, nq)):
        _check_token_tensor(name, t, p, n)
    _check_buffer("lse", lse, _torch().float32, p.batch * p.heads * nq)
    nqb, _, nnz = _block_counts(p)
    _check_selection(p, row_ptr, col_idx, nqb, nnz)
    for name, t, n in (("dq", dq, nq), ("dk", dk, nk), ("dv", dv, nk)):
        _on_device(name, t)
        if (t.dtype != _torch().float32 or not t.is_contiguous()
                or tuple(t.shape) != (p.batch, p.heads, n, p.head_dim)):
            raise ValueError(f"{name} must be contiguous fp32 [{p.batch}, {p.heads}, {n}, {p.head_dim}]")
    _check(load().lcsa_attn_bwd_noalloc(ctypes.byref(p), _ptr(q), _strides(q), _ptr(k), _strides(k), _ptr(v),
                                        _strides(v), _ptr(o), _strides(o), _ptr(d_o), _strides(d_o), _ptr(lse),
                                        _ptr(row_ptr), _ptr(col_idx), _ptr(dq), _ptr(dk), _ptr(dv),
                                        _stream(stream)))
    return dq, dk, dv


def forward(p: LcsaProblem, q, k, v, row_ptr=None, stream=None):
    """pool -> score_select -> attn_fwd on one stream. Returns a dict of device tensors."""
    torch = _torch()
    if row_ptr is None:
        row_ptr = torch.from_numpy(lcsa_csr_layout(p)[3]).to(q.device)
    qp, kp = lcsa_pool(p, q, k, stream=stream)
    col = lcsa_score_select(p, qp, kp, row_ptr, stream=stream)
    o, lse = lcsa_attn_fwd(p, q, k, v, row_ptr, col, stream=stream)
    return dict(q_pooled=qp, k_pooled=kp, row_ptr=row_ptr, col_idx=col, o=o, lse=lse)


# ------------------------------------------------------------------------------ streaming state
def lcsa_stream_state_size(chunk: LcsaProblem, cache_tblocks: int, ring_tblocks: int) -> int:
    n = ctypes.c_size_t()
    _check(load().lcsa_stream_state_size(ctypes.byref(chunk), cache_tblocks, ring_tblocks, ctypes.byref(n)))
    return n.value


class Stream:
    """Chunk-by-chunk LCSA with a K/V cache of the newest `cache_tblocks` temporal blocks (the C
    lcsa_stream_* calls; device memory from torch). `push(k_new, v_new)` appends one temporal block;
    `reserve()` gives the slot views a producer may write the next block into (then push those views:
    no copy); `window()` returns the current chunk's problem and K, V, pooled-K tensor views into the
    state; `forward(q)` runs lcsa_pool (q only) -> lcsa_score_select -> lcsa_attn_fwd on the window.
    ring_tblocks defaults to 2 * cache_tblocks - 1 slots (compaction every cache_tblocks pushes)."""

    def __init__(self, chunk: LcsaProblem, cache_tblocks: int, ring_tblocks: int = 0, device="cuda"):
        torch = _torch()
        self.chunk = chunk
        ring = ring_tblocks or max(1, 2 * cache_tblocks - 1)
        nbytes = lcsa_stream_state_size(chunk, cache_tblocks, ring)
        self.mem = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.state = LcsaStream()
        _check(load().lcsa_stream_init(ctypes.byref(self.state), ctypes.byref(chunk), cache_tblocks, ring,
                                       _ptr(self.mem), nbytes))
        self._rp = {}

    def _view(self, ptr, st: LcsaStrides, ntok: int):
        torch = _torch()
        dt = _dtype(self.chunk)
        esz = 4 if dt == torch.float32 else 2
        c = self.chunk
        return self.mem.view(dt).as_strided((c.batch, c.heads, ntok, c.head_dim), (st.batch, st.head, st.token, 1),
                                            (ptr - self.mem.data_ptr()) // esz)

    def reserve(self, stream=None):
        """(k_slot, v_slot): tensor views of the ring slot the next pushed block occupies."""
        kp, vp_ = ctypes.c_void_p(), ctypes.c_void_p()
        ks, vs = LcsaStrides(), LcsaStrides()
        _check(load().lcsa_stream_reserve(ctypes.byref(self.state), ctypes.byref(kp), ctypes.byref(ks),
                                          ctypes.byref(vp_), ctypes.byref(vs), _stream(stream)))
        n = 2 * self.chunk.grid_h * self.chunk.grid_w
        return self._view(kp.value, ks, n), self._view(vp_.value, vs, n)

    def push(self, k_new, v_new, stream=None):
        hw2 = 2 * self.chunk.grid_h * self.chunk.grid_w
        _check_token_tensor("k_new", k_new, self.chunk, hw2)
        _check_token_tensor("v_new", v_new, self.chunk, hw2)
        _check(load().lcsa_stream_push(ctypes.byref(self.state), _ptr(k_new), _strides(k_new), _ptr(v_new),
                                       _strides(v_new), _stream(stream)))

    def window(self):
        """(problem, k, v, k_pooled): tensor views into the state, valid until the next push."""
        torch = _torch()
        p = LcsaProblem()
        kp, vp_, kbp = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
        ks, vs = LcsaStrides(), LcsaStrides()
        _check(load().lcsa_stream_window(ctypes.byref(self.state), ctypes.byref(p), ctypes.byref(kp),
                                         ctypes.byref(ks), ctypes.byref(vp_), ctypes.byref(vs), ctypes.byref(kbp)))
        base = self.mem.data_ptr()
        nk = p.kv_frames * p.grid_h * p.grid_w
        k = self._view(kp.value, ks, nk)
        v = self._view(vp_.value, vs, nk)
        _, nkb, _, _ = lcsa_csr_layout(p)
        kbar = self.mem.view(torch.float32).as_strided((p.batch, p.heads, nkb, p.head_dim),
                                                       (p.heads * nkb * p.head_dim, nkb * p.head_dim, p.head_dim, 1),
                                                       (kbp.value - base) // 4)
        return p, k, v, kbar

    def forward(self, q, o=None, stream=None):
        """The newest chunk's attention: q [B, Hh, 2*H*W, d] are its query frames; o, if given, is
        the output view (any strides the C ABI accepts, e.g. a [B, N, Hh, d] buffer permuted)."""
        torch = _torch()
        p, k, v, kbar = self.window()
        key = p.kv_frames
        if key not in self._rp:
            self._rp[key] = torch.from_numpy(lcsa_csr_layout(p)[3]).to(q.device)
        row_ptr = self._rp[key]
        qp, _ = lcsa_pool(p, q, None, stream=stream)
        col = lcsa_score_select(p, qp, kbar, row_ptr, stream=stream)
        o, lse = lcsa_attn_fwd(p, q, k, v, row_ptr, col, o=o, stream=stream)
        return dict(problem=p, q_pooled=qp, k_pooled=kbar, row_ptr=row_ptr, col_idx=col, o=o, lse=lse)


# ---------------------------------------------------------------------------------- 3D RoPE
def lcsa_rope_qkv(p: LcsaProblem, rope: LcsaRope, qkv, frame0: int, q=None, k=None, v=None, stream=None):
    """qkv: bf16 [B, N, 3 * heads * head_dim] (rows [3][heads][d]) for latent frames
    [frame0, frame0 + N / (H*W)) -> rope(q), rope(k), v as [B, heads, N, d] tensors (given ones are
    written in place, e.g. the views of Stream.reserve())."""
    torch = _torch()
    hw = p.grid_h * p.grid_w
    if qkv.dim() != 3 or qkv.dtype != torch.bfloat16 or qkv.stride(2) != 1 or qkv.shape[0] != p.batch \
            or qkv.shape[2] != 3 * p.heads * p.head_dim or qkv.shape[1] % hw:
        raise ValueError("qkv must be bf16 [B, frames*H*W, 3*heads*head_dim] with unit last stride")
    _on_device("qkv", qkv)
    n = qkv.shape[1]
    outs = []
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is None:
            t = torch.empty((p.batch, p.heads, n, p.head_dim), dtype=torch.bfloat16, device=qkv.device)
        _check_token_tensor(name, t, p, n)
        outs.append(t)
    _check(load().lcsa_rope_qkv(ctypes.byref(p), ctypes.byref(rope), _ptr(qkv), qkv.stride(0), qkv.stride(1),
                                frame0, n // hw, _ptr(outs[0]), _strides(outs[0]), _ptr(outs[1]),
                                _strides(outs[1]), _ptr(outs[2]), _strides(outs[2]), _stream(stream)))
    return tuple(outs)


def lcsa_mfma_probe(workgroups: int, iters: int, sink, stream=None) -> float:
    """Launches the matrix-core throughput probe (measurement support, not part of the method) on
    `stream`; sink: fp32 device tensor of at least workgroups * 256 elements. Returns the FLOP the
    launch executes."""
    torch = _torch()
    _on_device("sink", sink)
    if sink.dtype != torch.float32 or not sink.is_contiguous() or sink.numel() < workgroups * 256:
        raise ValueError(f"sink must be a contiguous float32 device tensor of >= {workgroups * 256} elements")
    flop = ctypes.c_double(0.0)
    _check(load().lcsa_mfma_probe(workgroups, iters, _ptr(sink), ctypes.byref(flop), _stream(stream)))
    return flop.value
