"""Named LCSA problem shapes.

A workload is pure geometry and sizes: no arithmetic of the method lives here.
Shapes follow FlashVSR's streaming setting: 768x1408 output frames give a
48x88 latent token grid per latent frame, 1536x2688 give 96x168; a streaming
chunk is 8 video frames = 2 latent frames that attend causally to earlier
(cached) latent frames ("FlashVSR: Towards Real-time Diffusion-Based Streaming
Video Super Resolution", fmread summary, sec. 3 efficiency: 8-frame lookahead;
sec. 2.2 stage 2: 2x8x8 blocks; sec. 2.3: 1152x1152 locality window).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass

WIN_NONE, WIN_TRUNCATED, WIN_PRESERVING = 0, 1, 2
WIN_NAMES = {"none": WIN_NONE, "truncated": WIN_TRUNCATED, "preserving": WIN_PRESERVING}


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    heads: int
    head_dim: int
    grid_h: int          # latent tokens per frame, vertical
    grid_w: int          # latent tokens per frame, horizontal
    kv_frames: int       # K/V hold latent frames [0, kv_frames)
    q_frame0: int        # Q holds latent frames [q_frame0, q_frame0 + q_frames)
    q_frames: int
    dtype: str = "bf16"  # "bf16" or "f32" for Q/K/V/O
    win_mode: int = WIN_NONE
    win_h: int = 0       # tokens
    win_w: int = 0
    topk: int = 0        # > 0: fixed K per row; 0: use keep_ratio
    keep_ratio: float = 1.0
    blk_t: int = 2
    blk_h: int = 8
    blk_w: int = 8

    @property
    def scale(self) -> float:
        """Softmax scale 1/sqrt(head_dim), as the fp32 value passed to the kernels."""
        import numpy as np
        return float(np.float32(1.0 / np.sqrt(self.head_dim)))

    @property
    def nq_tokens(self) -> int:
        return self.q_frames * self.grid_h * self.grid_w

    @property
    def nk_tokens(self) -> int:
        return self.kv_frames * self.grid_h * self.grid_w

    @property
    def blocks_per_tblock(self) -> int:
        # a grid that is not a multiple of the block is cut from its origin; edge blocks are partial
        return (-(-self.grid_h // self.blk_h)) * (-(-self.grid_w // self.blk_w))

    @property
    def nqb(self) -> int:
        return (self.q_frames // self.blk_t) * self.blocks_per_tblock

    @property
    def nkb(self) -> int:
        return (self.kv_frames // self.blk_t) * self.blocks_per_tblock

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


RHO = 0.136  # keep ratio of the sparsity ablation (13.6% of blocks kept)

# Tiny case: T=4, 16x16 grid, 8 blocks, fixed top-3, fp32 I/O, d=64.
TINY = Workload("tiny_t4_16x16_h2_d64_f32", batch=1, heads=2, head_dim=64, grid_h=16, grid_w=16,
                kv_frames=4, q_frame0=0, q_frames=4, dtype="f32", topk=3)

# One 768x1408 streaming chunk: 2 query latent frames over 6 (4 cached + 2 current).
CHUNK_768 = Workload("chunk_768x1408_q2_kv6", batch=1, heads=12, head_dim=128, grid_h=48, grid_w=88,
                     kv_frames=6, q_frame0=4, q_frames=2, keep_ratio=RHO)

# One 720x1280 streaming chunk: 45x80 latent tokens (16 px per token), so the last block row is
# partial (5 of 8 token rows).
HD_720 = Workload("hd_720x1280_q2_kv6", batch=1, heads=12, head_dim=128, grid_h=45, grid_w=80,
                  kv_frames=6, q_frame0=4, q_frames=2, keep_ratio=RHO)

# Full-clip parallel (training-style) pass: 26 latent frames, block-causal.
CLIP_768 = Workload("clip_768x1408_26f", batch=1, heads=12, head_dim=128, grid_h=48, grid_w=88,
                    kv_frames=26, q_frame0=0, q_frames=26, keep_ratio=RHO)

# Ultra-high-resolution chunk at 1536x2688 with a 72x72-token (1152 px) locality window.
UHD_TRUNC = Workload("chunk_1536x2688_win72_truncated", batch=1, heads=12, head_dim=128,
                     grid_h=96, grid_w=168, kv_frames=6, q_frame0=4, q_frames=2,
                     win_mode=WIN_TRUNCATED, win_h=72, win_w=72, keep_ratio=RHO)
UHD_PRES = UHD_TRUNC.replace(name="chunk_1536x2688_win72_preserving", win_mode=WIN_PRESERVING)

# Sparsity sweep at the 768x1408 shape over 8 latent frames; rho = 1 is dense block-causal.
SWEEP_RHOS = (0.05, 0.136, 0.25, 0.5, 1.0)


def sweep(rho: float) -> Workload:
    return Workload(f"sweep_768x1408_8f_rho{rho:g}", batch=1, heads=12, head_dim=128, grid_h=48,
                    grid_w=88, kv_frames=8, q_frame0=0, q_frames=8, keep_ratio=rho)


ALL = [TINY, CHUNK_768, CLIP_768, UHD_TRUNC, UHD_PRES, HD_720] + [sweep(r) for r in SWEEP_RHOS]
BY_NAME = {w.name: w for w in ALL}
