"""Plain float64 CPU oracle of the Star Attention two-phase attention hot path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
library (``long_context_attention_amd``); the two meet only in the seeded input
generators of ``workloads``.

Every function follows a passage of the Star Attention pages (cited as
"page 1" = "Star Attention 完全拆解(一)", section titles in its own words) and is
written for readability, not speed: numpy float64, one library matmul per step,
no tiling, no fusion, no reordering beyond what the definition states.

Readings of the pages where they leave a step open:
  * RoPE is not printed. Rotate-half pairing (j, j+d/2), frequencies
    theta^(-2j/d), no frequency scaling; angles in float64.
  * The mask inside an augmented block is index-causal over [anchor, block]
    (an ordinary causal forward over the concatenation).
  * The LSE is the natural log of the sum of exp of the *scaled* scores.
  * GQA: query head h reads KV head floor(h / (Hq/Hkv)).
  * Query and generated tokens continue the positions at L, are appended to
    the query host's KV (the last host) and attend causally among themselves.
  * An empty (fully masked) partition has lse = -inf and weight 0.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
except the Star-vs-global deviation of context outputs in blocks >= 3, which
the pages only characterise through downstream task accuracy (parity unpinned,
reported as context only).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# RoPE (page 1, "repo implementation": positions are concatenated and only
# position differences matter under RoPE). Formula not printed on the pages.
# ---------------------------------------------------------------------------
def rope_inv_freq(head_dim: int, theta: float) -> np.ndarray:
    """Rotary frequencies theta^(-2j/d), j = 0..d/2-1 (float64)."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * j / head_dim)


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotate ``x`` [n, H, d] at integer positions ``pos`` [n] (rotate-half pairing)."""
    assert np.issubdtype(np.asarray(x).dtype, np.floating), "widen bf16 bit patterns first"
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_inv_freq(d, theta)[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# ---------------------------------------------------------------------------
# Softmax attention with explicit visibility (page 1, Phase 2 "local attention
# and local statistics": A_h = softmax(QK^T/sqrt(d)) V_h and s_h = sum exp).
# ---------------------------------------------------------------------------
def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, visible: np.ndarray,
              scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Softmax attention of ``q`` [nq,Hq,d] over ``k``/``v`` [nk,Hkv,d].

    ``visible`` [nq, nk] is True where the key may be attended. Returns the
    normalised output [nq,Hq,d] and lse = log(sum_k exp(scale*q.k)) [nq,Hq]
    over visible keys; a row that sees no key gets output 0 and lse -inf.
    """
    nq, hq, d = q.shape
    nk, hkv, _ = k.shape
    g = hq // hkv
    out = np.zeros((nq, hq, d), dtype=np.float64)
    lse = np.full((nq, hq), NEG_INF, dtype=np.float64)
    if nq == 0 or nk == 0:
        return out, lse
    vis = np.asarray(visible, dtype=bool)
    for kh in range(hkv):
        qh = q[:, kh * g:(kh + 1) * g, :].reshape(nq * g, d)
        s = scale * (qh @ k[:, kh, :].T)                      # [nq*g, nk]
        s = s.reshape(nq, g, nk)
        s = np.where(vis[:, None, :], s, NEG_INF)
        m = s.max(axis=-1)                                    # [nq, g]
        m_ref = np.where(np.isfinite(m), m, 0.0)
        e = np.exp(s - m_ref[..., None])                      # masked -> exp(-inf) = 0
        z = e.sum(axis=-1)                                    # [nq, g]
        num = (e.reshape(nq * g, nk) @ v[:, kh, :]).reshape(nq, g, d)
        with np.errstate(divide="ignore", invalid="ignore"):
            o = np.where(z[..., None] > 0, num / z[..., None], 0.0)
            l_ = np.where(z > 0, m_ref + np.log(z), NEG_INF)
        out[:, kh * g:(kh + 1) * g, :] = o
        lse[:, kh * g:(kh + 1) * g] = l_
    return out, lse


# ---------------------------------------------------------------------------
# Phase 1 (page 1, "Phase 1: augmented context", "local attention and KV
# discard", and the quoted _process_blockwise_context excerpt).
# ---------------------------------------------------------------------------
ANCHORS = ("first", "previous")


def augmented_block(i: int, block_len: int, anchor_len: int, anchor: str = "first") -> tuple[np.ndarray, int]:
    """Token indices of augmented block c'_i (1-based i) and its anchor length.

    c'_1 = c_1; for i > 1, c'_i = (first ``anchor_len`` tokens of the anchor
    block, c_i). The anchor block is c_1 (the method), or with
    ``anchor="previous"`` the block just before c_i, c_{i-1} (the ablation the
    paper ran against it, page 1, section on vLLM's chunked local attention
    backend). Positions equal the token indices: the anchor keeps its own
    positions and block i keeps [(i-1)b, ib). For i = 2 both anchors are c_1.
    """
    assert anchor in ANCHORS, anchor
    blk = np.arange((i - 1) * block_len, i * block_len)
    if i == 1:
        return blk, 0
    a0 = 0 if anchor == "first" else (i - 2) * block_len
    return np.concatenate([np.arange(a0, a0 + anchor_len), blk]), anchor_len


def augmented_positions(i: int, block_len: int, anchor_len: int, anchor: str = "first",
                        anchor_pos=None) -> np.ndarray:
    """Position IDs of the tokens of c'_i (same order as ``augmented_block``).

    By default every token keeps its own position (page 1, "problem
    definition": the anchor keeps [0, b), block i keeps [(i-1)b, ib)). The
    paper's position ablation (page 3, section 4.1 on the anchor block's
    position and content; page 1, "scope and engineering notes") gives the
    anchor other position IDs, e.g. drawn at random from the prefix or placed
    right before the block: with ``anchor_pos`` (one entry per block, entry i-1 for
    c'_i, entry 0 unused) the anchor tokens of c'_i sit at consecutive
    positions anchor_pos[i-1], anchor_pos[i-1] + 1, ...; block i keeps its own.
    """
    tok, n_anc = augmented_block(i, block_len, anchor_len, anchor)
    pos = tok.copy()
    if anchor_pos is not None and n_anc:
        pos[:n_anc] = int(anchor_pos[i - 1]) + np.arange(n_anc)
    return pos


def phase1_block(q_ctx, k_ctx, v_ctx, i: int, block_len: int, anchor_len: int,
                 theta: float, scale: float, rows=None, with_anchor_rows: bool = False,
                 anchor: str = "first", anchor_pos=None) -> dict:
    """Literal Phase 1 for augmented block i.

    Runs ordinary index-causal attention over c'_i at its positions (see
    ``augmented_positions``), keeps the outputs of block rows ``rows`` (offsets
    inside c_i; default all), and the block's own RoPE'd K and V (the anchor's
    KV is discarded).
    """
    tok, n_anc = augmented_block(i, block_len, anchor_len, anchor)
    pos = augmented_positions(i, block_len, anchor_len, anchor, anchor_pos)
    rows = np.arange(block_len) if rows is None else np.asarray(rows)
    sel = n_anc + rows                                        # augmented indices of wanted rows
    if with_anchor_rows and n_anc:
        sel = np.concatenate([np.arange(n_anc), sel])
    n_keys = int(sel.max()) + 1
    ktok = tok[:n_keys]
    k = rope(k_ctx[ktok], pos[:n_keys], theta)
    v = np.asarray(v_ctx[ktok], dtype=np.float64)
    q = rope(q_ctx[tok[sel]], pos[sel], theta)
    visible = np.arange(n_keys)[None, :] <= sel[:, None]      # index-causal over c'_i
    out, _ = attention(q, k, v, visible, scale)
    res = {"rows": rows, "out": out[-len(rows):] if len(rows) else out[:0]}
    if with_anchor_rows and n_anc:
        res["anchor_out"] = out[:n_anc]
    if n_keys > n_anc:
        res["k_block"] = k[n_anc:]
        res["v_block"] = v[n_anc:]
    return res


def phase1(q_ctx, k_ctx, v_ctx, block_len: int, anchor_len: int, theta: float, scale: float,
           rows_by_block: dict | None = None, anchor: str = "first", anchor_pos=None) -> dict:
    """Literal Phase 1 over all blocks.

    Returns ``out`` {block i: [rows, Hq, d]}, ``rows`` {i: offsets} and the KV
    cache ``k_cache``/``v_cache`` [L, Hkv, d] assembled from each block's
    non-anchor KV. With ``rows_by_block`` only those rows' outputs are computed
    (the cache is then built from a separate, cheaper pass per block).
    ``anchor`` selects the anchor block as in ``augmented_block`` and
    ``anchor_pos`` its position IDs as in ``augmented_positions``.
    """
    L = q_ctx.shape[0]
    n = L // block_len
    outs, rows_out = {}, {}
    k_cache = np.empty((L,) + k_ctx.shape[1:], dtype=np.float64)
    v_cache = np.empty_like(k_cache)
    for i in range(1, n + 1):
        rows = None if rows_by_block is None else rows_by_block[i]
        res = phase1_block(q_ctx, k_ctx, v_ctx, i, block_len, anchor_len, theta, scale, rows, anchor=anchor,
                           anchor_pos=anchor_pos)
        outs[i], rows_out[i] = res["out"], res["rows"]
        blk = slice((i - 1) * block_len, i * block_len)
        if "k_block" in res and res["k_block"].shape[0] == block_len:
            k_cache[blk], v_cache[blk] = res["k_block"], res["v_block"]
        else:  # sampled rows did not reach the end of the block: KV of c_i at its positions
            tok = np.arange(blk.start, blk.stop)
            k_cache[blk] = rope(k_ctx[tok], tok, theta)
            v_cache[blk] = v_ctx[tok]
    return {"out": outs, "rows": rows_out, "k_cache": k_cache, "v_cache": v_cache}


def exact_causal(q_ctx, k_ctx, v_ctx, theta: float, scale: float, rows=None) -> np.ndarray:
    """Exact global causal attention of context rows over all earlier context tokens."""
    L = q_ctx.shape[0]
    rows = np.arange(L) if rows is None else np.asarray(rows)
    n_keys = int(rows.max()) + 1
    tok = np.arange(n_keys)
    k = rope(k_ctx[:n_keys], tok, theta)
    q = rope(q_ctx[rows], rows, theta)
    visible = tok[None, :] <= rows[:, None]
    out, _ = attention(q, k, np.asarray(v_ctx[:n_keys], dtype=np.float64), visible, scale)
    return out


# ---------------------------------------------------------------------------
# Phase 2 (page 1, "Phase 2: global attention and distributed softmax",
# "assembling the global result", "numerical stability: log-sum-exp",
# "query-host logic").
# ---------------------------------------------------------------------------
def tail_keys(k_new_pre, v_new, pos0: int, theta: float) -> tuple[np.ndarray, np.ndarray]:
    """KV of query / generated tokens held by the query host, RoPE'd at pos0.."""
    pos = pos0 + np.arange(k_new_pre.shape[0])
    return rope(k_new_pre, pos, theta), np.asarray(v_new, dtype=np.float64)


def phase2_partials(q_pre, q_pos0: int, k_cache, v_cache, block_len: int,
                    k_tail, v_tail, tail_pos0: int, theta: float, scale: float):
    """Local attention of every partition (context blocks 1..n, then the tail).

    Query token t sits at position q_pos0 + t. A key is visible iff its position
    does not exceed the query's. Returns out_part [n+1, T, Hq, d] (each A_h
    normalised over its own keys) and lse_part [n+1, T, Hq].
    """
    T = q_pre.shape[0]
    qpos = q_pos0 + np.arange(T)
    q = rope(q_pre, qpos, theta)
    L = k_cache.shape[0]
    n = L // block_len
    parts = [(k_cache[(j - 1) * block_len: j * block_len], v_cache[(j - 1) * block_len: j * block_len],
              np.arange((j - 1) * block_len, j * block_len)) for j in range(1, n + 1)]
    parts.append((k_tail, v_tail, tail_pos0 + np.arange(k_tail.shape[0])))
    outs, lses = [], []
    for kj, vj, kpos in parts:
        visible = kpos[None, :] <= qpos[:, None]
        o, l_ = attention(q, kj, vj, visible, scale)
        outs.append(o)
        lses.append(l_)
    return np.stack(outs), np.stack(lses)


def merge(out_part: np.ndarray, lse_part: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Global aggregation of the partials.

    s_global = sum_h s_h and A_global = sum_h (s_h / s_global) A_h, carried in
    LSE form with the largest lse subtracted first so nothing overflows; a
    partition with lse = -inf has weight 0, and if every partition is empty the
    result is output 0, lse -inf.
    """
    m = lse_part.max(axis=0)                                  # [T, Hq]
    m_ref = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lse_part - m_ref[None])                        # s_h / exp(M)
    s = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(s[..., None] > 0, (w[..., None] * out_part).sum(axis=0) / s[..., None], 0.0)
        lse = np.where(s > 0, m_ref + np.log(s), NEG_INF)
    return out, lse


def merge_pairwise_literal(out_part: np.ndarray, lse_part: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """The pages' sequential pairwise update, written as printed (no max guard).

    lse_new = lse_old + log(1 + exp(lse_b - lse_old));
    out_new = exp(lse_old - lse_new) out_old + exp(lse_b - lse_new) out_b.
    Kept only to show agreement on benign inputs and the overflow hazard the
    pages warn about; ``merge`` is the oracle's merge.
    """
    out, lse = out_part[0].copy(), lse_part[0].copy()
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        for j in range(1, out_part.shape[0]):
            lse_new = lse + np.log(1.0 + np.exp(lse_part[j] - lse))
            out = np.exp(lse - lse_new)[..., None] * out + np.exp(lse_part[j] - lse_new)[..., None] * out_part[j]
            lse = lse_new
    return out, lse


def phase2_plain(q_pre, q_pos0: int, k_cache, v_cache, k_tail, v_tail, tail_pos0: int,
                 theta: float, scale: float):
    """Softmax attention of the query rows over the concatenation of every cached key."""
    T = q_pre.shape[0]
    qpos = q_pos0 + np.arange(T)
    q = rope(q_pre, qpos, theta)
    k = np.concatenate([k_cache, k_tail])
    v = np.concatenate([v_cache, v_tail])
    kpos = np.concatenate([np.arange(k_cache.shape[0]), tail_pos0 + np.arange(k_tail.shape[0])])
    return attention(q, k, v, kpos[None, :] <= qpos[:, None], scale)

