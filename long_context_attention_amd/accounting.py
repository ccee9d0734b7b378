"""Work and traffic accounting for the Star Attention hot path (host-side counting only).

Useful work counts what the method needs, not what a kernel happens to do:
  * Phase 1 counts unmasked (query row, key) pairs per query head. Block 1 is
    plain causal attention over its b tokens; every other block's rows attend to
    the whole anchor and to their causal prefix inside the block (Star Attention
    pages, page 1, "Phase 1: augmented context"). Anchor rows are not counted:
    their outputs equal block 1's first A rows, so they are never recomputed.
    FLOPs = 4 * head_dim * n_q_heads * pairs (QK^T and PV, 2 FLOP per MAC).
  * Phase 2 counts the bytes a step must move: every visible cached K and V row
    (context cache plus the query host's tail), the query rows read and the
    merged output written. Per-partition partials are an implementation detail
    and are not counted.
  * The sizing helpers restate the pages' own arithmetic (page 1, "cost of long
    context" and "communication volume") so tests can pin this module to it.
"""
from __future__ import annotations


def phase1_pairs(ctx_len: int, block_len: int, anchor_len: int) -> int:
    n = ctx_len // block_len
    b = block_len
    causal = b * (b + 1) // 2
    return causal + (n - 1) * (b * anchor_len + causal)


def phase1_flops(ctx_len: int, block_len: int, anchor_len: int, n_q_heads: int, head_dim: int) -> int:
    return 4 * head_dim * n_q_heads * phase1_pairs(ctx_len, block_len, anchor_len)


def phase1_recompute_flops(ctx_len: int, block_len: int, anchor_len: int, n_q_heads: int, head_dim: int) -> int:
    """FLOPs if every augmented block were run whole, anchor rows included (the pages' form)."""
    n = ctx_len // block_len
    b, a = block_len, anchor_len
    aug = (a + b) * (a + b + 1) // 2
    return 4 * head_dim * n_q_heads * (b * (b + 1) // 2 + (n - 1) * aug)


def global_causal_flops(ctx_len: int, n_q_heads: int, head_dim: int) -> int:
    return 4 * head_dim * n_q_heads * (ctx_len * (ctx_len + 1) // 2)


def phase2_step_bytes(ctx_len: int, tail_len: int, t_q: int, n_q_heads: int, n_kv_heads: int,
                      head_dim: int, elem_bytes: int) -> int:
    """Algorithmic HBM bytes of one Phase-2 step (query step or one decode step).

    ``tail_len`` is the number of tail rows after this step's append; every
    cached row is visible to the step's last token.
    """
    kv = 2 * (ctx_len + tail_len) * n_kv_heads * head_dim * elem_bytes
    q = t_q * n_q_heads * head_dim * elem_bytes
    out = t_q * n_q_heads * head_dim * elem_bytes + t_q * n_q_heads * 4   # output + fp32 lse
    return kv + q + out


def phase2_step_flops(ctx_len: int, tail_len: int, t_q: int, n_q_heads: int, head_dim: int) -> int:
    """Useful FLOPs of one Phase-2 step: token t sees ctx_len + tail_len - (t_q - 1 - t) keys."""
    keys = sum(ctx_len + tail_len - (t_q - 1 - t) for t in range(t_q))
    return 4 * head_dim * n_q_heads * keys


def kv_bytes_per_token(n_layers: int, n_kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V of one token across all layers."""
    return 2 * n_layers * n_kv_heads * head_dim * elem_bytes


def phase2_message_bytes(n_hosts: int, n_layers: int, n_tokens: int, n_heads: int, head_dim: int,
                         elem_bytes: int) -> int:
    """Phase-2 traffic: each host returns one vector and one scalar per head, layer and token."""
    return n_hosts * n_layers * n_tokens * n_heads * (head_dim + 1) * elem_bytes
