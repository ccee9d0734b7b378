"""Device buffers of one Star Attention layer and the order of the C calls.

``StarLayer`` owns (through PyTorch allocations) the Phase-1 output, the KV
cache, the query host's tail, the Phase-2 workspace and partials. ``encode``
runs Phase 1; ``step`` runs one Phase-2 step (the query step or a decode step):
append the new tokens' KV to the tail, local attention of every partition,
global merge. Every step of the computation runs in libstarattn.
"""
from __future__ import annotations

import torch

from . import _binding as B

TORCH_DTYPE = {B.SA_F32: torch.float32, B.SA_BF16: torch.bfloat16}


class StarLayer:
    def __init__(self, n_q_heads: int, n_kv_heads: int, head_dim: int, dtype: int, rope_theta: float,
                 softmax_scale: float, ctx_len: int, block_len: int, anchor_len: int, tail_cap: int,
                 max_t_q: int, device: str = "cuda", anchor_kind: int = B.SA_ANCHOR_FIRST, anchor_pos=None):
        self.desc = B.make_desc(n_q_heads, n_kv_heads, head_dim, dtype, rope_theta, softmax_scale)
        self.dtype = dtype
        self.tdtype = TORCH_DTYPE[dtype]
        self.hq, self.hkv, self.d = n_q_heads, n_kv_heads, head_dim
        self.L, self.b, self.A = ctx_len, block_len, anchor_len
        self.anchor_kind = anchor_kind
        # anchor position IDs per block (sa_phase1_encode_anchor_at), with the
        # workspace for the anchor's rotated keys
        self.anchor_pos = None if anchor_pos is None else [int(p) for p in anchor_pos]
        self.anchor_ws = None
        if self.anchor_pos is not None:
            nb = B.sa_anchor_at_workspace_bytes(self.desc, ctx_len, block_len, anchor_len)
            self.anchor_ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=device)
        # Phase 1's optional workspace: the job counters of its run-time job order
        self.p1_ws = torch.empty(max(B.sa_workspace_bytes(B.SA_CALL_PHASE1, self.desc, ctx_len, block_len, 1, 0), 16),
                                 dtype=torch.uint8, device=device)
        self.tail_cap = tail_cap
        self.tail_len = 0
        self.n_parts = ctx_len // block_len + 1
        self.device = device
        kw = dict(device=device, dtype=self.tdtype)
        self.out_ctx = torch.empty(ctx_len, n_q_heads, head_dim, **kw)
        self.k_cache = torch.empty(n_kv_heads, ctx_len, head_dim, **kw)
        self.v_cache = torch.empty(n_kv_heads, ctx_len, head_dim, **kw)
        self.k_tail = torch.zeros(n_kv_heads, max(tail_cap, 1), head_dim, **kw)
        self.v_tail = torch.zeros(n_kv_heads, max(tail_cap, 1), head_dim, **kw)
        ws = max(B.sa_workspace_bytes(B.SA_CALL_PHASE2, self.desc, ctx_len, block_len, t, tail_cap)
                 for t in sorted({1, max_t_q}))
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=device)
        # flat storage so that the partials of a t-row step are one dense [n_parts, t, ...] view
        self._out_part = torch.empty(self.n_parts * max_t_q * n_q_heads * head_dim, dtype=torch.float32,
                                     device=device)
        self._lse_part = torch.empty(self.n_parts * max_t_q * n_q_heads, dtype=torch.float32, device=device)
        self.out = torch.empty(max_t_q, n_q_heads, head_dim, **kw)
        self.lse = torch.empty(max_t_q, n_q_heads, dtype=torch.float32, device=device)

    @classmethod
    def for_workload(cls, w, max_t_q: int | None = None, device: str = "cuda", anchor_pos=None) -> "StarLayer":
        dt = B.SA_F32 if w.dtype == "f32" else B.SA_BF16
        return cls(w.n_q_heads, w.n_kv_heads, w.head_dim, dt, w.rope_theta, w.softmax_scale, w.ctx_len,
                   w.block_len, w.anchor_len, w.tail_cap, max_t_q or max(w.n_query, 1), device,
                   B.SA_ANCHOR_PREVIOUS if getattr(w, "anchor", "first") == "previous" else B.SA_ANCHOR_FIRST,
                   anchor_pos)

    def encode(self, q_ctx, k_ctx, v_ctx, stream=None) -> None:
        """Phase 1: cache the context KV and compute every context token's output."""
        if self.anchor_pos is not None:
            B.sa_phase1_encode_anchor_at(self.desc, self.L, self.b, self.A, self.anchor_pos, q_ctx, k_ctx, v_ctx,
                                         self.out_ctx, self.k_cache, self.v_cache, self.anchor_ws, stream)
        elif self.anchor_kind == B.SA_ANCHOR_FIRST:
            B.sa_phase1_encode(self.desc, self.L, self.b, self.A, q_ctx, k_ctx, v_ctx, self.out_ctx, self.k_cache,
                               self.v_cache, self.p1_ws, stream)
        else:
            B.sa_phase1_encode_anchor(self.desc, self.L, self.b, self.A, self.anchor_kind, q_ctx, k_ctx, v_ctx,
                                      self.out_ctx, self.k_cache, self.v_cache, self.p1_ws, stream)
        self.tail_len = 0

    def step(self, q, k_new, v_new, stream=None):
        """One Phase-2 step for t new tokens at positions L + tail_len ...; returns (out, lse, partials)."""
        t = q.shape[0]
        pos0 = self.L + self.tail_len
        B.sa_decode_append(self.desc, k_new, v_new, t, pos0, self.k_tail, self.v_tail, self.tail_cap,
                           self.tail_len, stream)
        self.tail_len += t
        n = self.n_parts * t * self.hq
        out_part = self._out_part[: n * self.d].view(self.n_parts, t, self.hq, self.d)
        lse_part = self._lse_part[:n].view(self.n_parts, t, self.hq)
        B.sa_phase2_partial(self.desc, q, t, pos0, self.k_cache, self.v_cache, self.L, self.b, self.k_tail,
                            self.v_tail, self.tail_cap, self.tail_len, self.L, out_part, lse_part, self.workspace,
                            stream)
        out, lse = self.out[:t], self.lse[:t]
        B.sa_phase2_merge(self.n_parts, t, self.hq, self.d, out_part, lse_part, out, self.dtype, lse, stream)
        return out, lse, out_part, lse_part

    def step_fused(self, q, k_new, v_new, stream=None):
        """The same step through sa_phase2_step (one call, three launches); returns (out, lse)."""
        t = q.shape[0]
        out, lse = self.out[:t], self.lse[:t]
        B.sa_phase2_step(self.desc, q, k_new, v_new, t, self.k_cache, self.v_cache, self.L, self.b, self.k_tail,
                         self.v_tail, self.tail_cap, self.tail_len, out, lse, self.workspace, stream)
        self.tail_len += t
        return out, lse
