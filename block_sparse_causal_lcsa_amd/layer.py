"""A DiT self-attention layer around streaming LCSA, with random weights: the workload that measures
LCSA's share of a Wan-shaped attention layer (FlashVSR summary, sec. 2.2 Stage 1 names the Wan2.1
DiT; sec. 3 attributes the runtime to its attention).

Per chunk (one temporal block of latent tokens, x: [B, 2*H*W, C], C = heads * head_dim):
  qkv = x @ Wqkv                          plain library GEMM (torch / hipBLASLt), bf16
  lcsa_rope_qkv                           3D RoPE of q and k, head split; k and v go straight into
                                          the stream's reserved ring slot (no copy on push)
  lcsa_stream_push                        pools the new K block into the pooled-K cache
  lcsa_pool(q) -> lcsa_score_select -> lcsa_attn_fwd on the stream window, O written as [B, N, C]
  out = O @ Wo                            plain library GEMM
Only the two projections run outside the library's kernels.
"""
from __future__ import annotations

import numpy as np

from . import lcsa


class DitLcsaLayer:
    def __init__(self, chunk: lcsa.LcsaProblem, cache_tblocks: int, rope_dims=(44, 42, 42), theta=10000.0,
                 seed=0, device="cuda", ring_tblocks: int = 0):
        import torch
        self.p = chunk
        self.C = chunk.heads * chunk.head_dim
        self.rope = lcsa.LcsaRope(*rope_dims, theta)
        g = torch.Generator(device="cpu").manual_seed(seed)
        std = 1.0 / np.sqrt(self.C)
        self.w_qkv = (torch.randn(self.C, 3 * self.C, generator=g) * std).to(torch.bfloat16).to(device)
        self.w_o = (torch.randn(self.C, self.C, generator=g) * std).to(torch.bfloat16).to(device)
        self.stream = lcsa.Stream(chunk, cache_tblocks, ring_tblocks, device=device)
        self.frame = 0  # absolute latent frame of the next chunk

    def step(self, x, stream=None, timing=None):
        """x: bf16 [B, 2*H*W, C] of the next chunk -> (out [B, 2*H*W, C], LCSA outputs).
        timing: optional list of 6 CUDA events recorded between the stages."""
        import torch
        p = self.p
        B, N, C = x.shape
        s = torch.cuda.current_stream() if stream is None else stream

        def mark(i):
            if timing is not None:
                timing[i].record(s)

        mark(0)
        qkv = torch.matmul(x.view(B * N, C), self.w_qkv).view(B, N, 3 * C)
        mark(1)
        k_slot, v_slot = self.stream.reserve(stream=s)
        q = torch.empty((B, p.heads, N, p.head_dim), dtype=torch.bfloat16, device=x.device)
        lcsa.lcsa_rope_qkv(p, self.rope, qkv, self.frame, q, k_slot, v_slot, stream=s)
        mark(2)
        self.stream.push(k_slot, v_slot, stream=s)
        mark(3)
        o = torch.empty((B, N, p.heads, p.head_dim), dtype=torch.bfloat16, device=x.device)
        res = self.stream.forward(q, o=o.permute(0, 2, 1, 3), stream=s)
        mark(4)
        out = torch.matmul(o.view(B * N, C), self.w_o).view(B, N, C)
        mark(5)
        self.frame += 2
        res.update(q=q, qkv=qkv, o_tokens=o)
        return out, res
