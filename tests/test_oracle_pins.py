"""Pins of the fp64 oracle against what the Star Attention pages and mathematics fix.

None of these tests needs a GPU. Each pin checks the oracle against something
other than itself: a library routine (torch's CPU float64 SDPA, numpy complex
arithmetic, scipy's logsumexp), a closed form, an invariant the pages state,
or an independent brute-force loop on tiny inputs.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle as O
from long_context_attention_amd import accounting as acc
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _torch_sdpa(q, k, v, visible, scale):
    """Library reference: torch CPU float64 SDPA with GQA expanded, plus logsumexp."""
    nq, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)                      # [Hq, nq, d]
    kt = torch.from_numpy(np.repeat(k, g, axis=1)).permute(1, 0, 2).contiguous()
    vt = torch.from_numpy(np.repeat(v, g, axis=1)).permute(1, 0, 2).contiguous()
    mask = torch.from_numpy(np.asarray(visible, dtype=bool))
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    s = scale * torch.einsum("hqd,hkd->hqk", qt, kt)
    s = s.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return out.permute(1, 0, 2).numpy(), lse.permute(1, 0).numpy()


# ----------------------------------------------------------------------------- RoPE
def test_rope_inv_freq_closed_form():
    f = O.rope_inv_freq(64, 1.0e4)
    assert f[0] == 1.0
    assert math.isclose(f[16], 1.0e4 ** -0.5, rel_tol=1e-15)
    assert math.isclose(f[1], 1.0e4 ** (-1.0 / 32.0), rel_tol=1e-15)
    assert np.all(np.diff(f) < 0)


def test_rope_matches_complex_rotation(rng):
    # rotate-half pairing: element j pairs with j + d/2; (x_j + i x_{j+d/2}) * exp(i p theta_j)
    x = _rand(rng, 7, 3, 16)
    pos = rng.integers(0, 100000, size=7)
    theta = 5.0e5
    got = O.rope(x, pos, theta)
    z = x[..., :8] + 1j * x[..., 8:]
    j = np.arange(8)
    rot = np.exp(1j * pos[:, None, None] * theta ** (-2.0 * j / 16.0))
    want = z * rot
    np.testing.assert_allclose(got[..., :8], want.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[..., 8:], want.imag, rtol=0, atol=1e-12)


def test_rope_identity_norm_group_and_relative(rng):
    x = _rand(rng, 5, 2, 32)
    np.testing.assert_array_equal(O.rope(x, np.zeros(5, dtype=int), 1e4), x)
    y = O.rope(x, np.arange(5) * 977, 1e4)
    np.testing.assert_allclose(x[..., :16] ** 2 + x[..., 16:] ** 2, y[..., :16] ** 2 + y[..., 16:] ** 2, atol=1e-12)
    # group property: rotating by p1 then p2 equals rotating by p1 + p2
    p1, p2 = np.arange(5) * 13, np.arange(5) * 4099 + 7
    np.testing.assert_allclose(O.rope(O.rope(x, p1, 1e4), p2, 1e4), O.rope(x, p1 + p2, 1e4), atol=1e-10)
    # relative property: q(p).k(p') depends only on p - p'
    q, k = _rand(rng, 1, 1, 32), _rand(rng, 1, 1, 32)
    for shift in (0, 1, 1000, 999_983):
        a = O.rope(q, np.array([500 + shift]), 5e5).ravel() @ O.rope(k, np.array([123 + shift]), 5e5).ravel()
        b = O.rope(q, np.array([500]), 5e5).ravel() @ O.rope(k, np.array([123]), 5e5).ravel()
        assert abs(a - b) < 1e-9


# ----------------------------------------------------------------------------- attention
def test_attention_matches_torch_sdpa(rng):
    q, k, v = _rand(rng, 9, 4, 16), _rand(rng, 13, 2, 16), _rand(rng, 13, 2, 16)
    visible = rng.random((9, 13)) < 0.6
    visible[:, 0] = True
    out, lse = O.attention(q, k, v, visible, 0.3)
    ro, rl = _torch_sdpa(q, k, v, visible, 0.3)
    np.testing.assert_allclose(out, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)


def test_attention_special_inputs(rng):
    nq, nk, d = 4, 10, 8
    q, k = _rand(rng, nq, 2, d), _rand(rng, nk, 1, d)
    vis = np.tril(np.ones((nq, nk), dtype=bool), k=3)           # row r sees keys 0..r+3
    # constant V -> output is that constant
    vc = np.full((nk, 1, d), 2.5)
    out, _ = O.attention(q, k, vc, vis, 0.7)
    np.testing.assert_allclose(out, 2.5, atol=1e-13)
    # K = 0 -> uniform weights: output = mean of visible V, lse = log(#visible)
    v = _rand(rng, nk, 1, d)
    out, lse = O.attention(q, np.zeros_like(k), v, vis, 0.7)
    for r in range(nq):
        n_vis = r + 4
        np.testing.assert_allclose(out[r, 0], v[:n_vis, 0].mean(axis=0), atol=1e-13)
        np.testing.assert_allclose(lse[r], math.log(n_vis), atol=1e-13)
    # a single visible key -> that key's V; lse = its scaled score
    one = np.zeros((nq, nk), dtype=bool)
    one[:, 5] = True
    out, lse = O.attention(q, k, v, one, 0.7)
    np.testing.assert_allclose(out[:, 1], np.broadcast_to(v[5, 0], (nq, d)), atol=1e-13)
    np.testing.assert_allclose(lse[:, 1], 0.7 * q[:, 1] @ k[5, 0], atol=1e-13)
    # no visible key -> output 0 and lse -inf (never NaN)
    out, lse = O.attention(q, k, v, np.zeros((nq, nk), dtype=bool), 0.7)
    assert np.all(out == 0) and np.all(lse == -np.inf)


# ----------------------------------------------------------------------------- Phase 1
def _ctx(rng, L, hq, hkv, d):
    return _rand(rng, L, hq, d), _rand(rng, L, hkv, d), _rand(rng, L, hkv, d)


def test_phase1_single_block_is_exact_causal(rng):
    """With n = 1 block, c' = c_1 and Phase 1 is ordinary causal attention."""
    L, theta, scale = 48, 1e4, 0.25
    q, k, v = _ctx(rng, L, 4, 2, 16)
    res = O.phase1(q, k, v, L, L, theta, scale)
    pos = np.arange(L)
    ro, _ = _torch_sdpa(O.rope(q, pos, theta), O.rope(k, pos, theta), v,
                        np.tril(np.ones((L, L), dtype=bool)), scale)
    np.testing.assert_allclose(res["out"][1], ro, atol=1e-12)


def test_phase1_blocks_one_and_two_are_exact(rng):
    """Block 1 has no anchor; block 2's augmented sequence is the true prefix."""
    L, b, theta, scale = 64, 16, 1e4, 0.25
    q, k, v = _ctx(rng, L, 2, 1, 8)
    res = O.phase1(q, k, v, b, b, theta, scale)
    ex = O.exact_causal(q, k, v, theta, scale)
    np.testing.assert_allclose(res["out"][1], ex[:b], atol=1e-12)
    np.testing.assert_allclose(res["out"][2], ex[b:2 * b], atol=1e-12)
    # blocks >= 3 really are approximations (otherwise the pins above prove nothing)
    assert np.abs(res["out"][3] - ex[2 * b:3 * b]).max() > 1e-3


def _brute_phase1(q, k, v, b, A, theta, scale):
    """Independent loop form of Phase 1 on tiny inputs (complex-number RoPE, math.exp)."""
    L, hq, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    h2 = d // 2

    def rot(x, p):
        out = np.empty(d)
        for j in range(h2):
            z = complex(x[j], x[j + h2]) * complex(math.cos(p * theta ** (-2 * j / d)),
                                                   math.sin(p * theta ** (-2 * j / d)))
            out[j], out[j + h2] = z.real, z.imag
        return out

    out = np.zeros_like(q)
    for i in range(1, L // b + 1):
        toks = list(range((i - 1) * b, i * b)) if i == 1 else list(range(A)) + list(range((i - 1) * b, i * b))
        n_anc = 0 if i == 1 else A
        for r in range(b):
            a_idx = n_anc + r
            for h in range(hq):
                qv = rot(q[toks[a_idx], h], toks[a_idx])
                scores = []
                for j in range(a_idx + 1):
                    kv = rot(k[toks[j], h // g], toks[j])
                    scores.append(scale * sum(qv[t] * kv[t] for t in range(d)))
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = sum(w)
                for j in range(a_idx + 1):
                    out[toks[a_idx], h] += (w[j] / tot) * v[toks[j], h // g]
    return out


@pytest.mark.parametrize("A", [2, 1])
def test_phase1_brute_force_tiny(rng, A):
    L, b, theta, scale = 8, 2, 10.0, 0.5
    q, k, v = _ctx(rng, L, 2, 1, 4)
    res = O.phase1(q, k, v, b, A, theta, scale)
    got = np.concatenate([res["out"][i] for i in range(1, L // b + 1)])
    np.testing.assert_allclose(got, _brute_phase1(q, k, v, b, A, theta, scale), atol=1e-12)


def test_phase1_equals_anchor_plus_block_merge(rng):
    """Second form: merge(anchor attention unmasked, in-block causal by position) == literal c'_i."""
    L, b, A, theta, scale = 96, 24, 17, 1e4, 0.3
    q, k, v = _ctx(rng, L, 4, 2, 16)
    res = O.phase1(q, k, v, b, A, theta, scale)
    for i in range(2, L // b + 1):
        blk = np.arange((i - 1) * b, i * b)
        anc = np.arange(A)
        qr = O.rope(q[blk], blk, theta)
        o_a, l_a = O.attention(qr, O.rope(k[anc], anc, theta), v[anc], np.ones((b, A), dtype=bool), scale)
        o_b, l_b = O.attention(qr, O.rope(k[blk], blk, theta), v[blk], blk[None, :] <= blk[:, None], scale)
        o, _ = O.merge(np.stack([o_a, o_b]), np.stack([l_a, l_b]))
        np.testing.assert_allclose(o, res["out"][i], atol=1e-12)


def test_phase1_anchor_rows_equal_block1(rng):
    """Anchor rows of every augmented block reproduce block 1's first A rows."""
    L, b, A, theta, scale = 60, 20, 13, 1e4, 0.3
    q, k, v = _ctx(rng, L, 2, 2, 8)
    first = O.phase1_block(q, k, v, 1, b, A, theta, scale)["out"][:A]
    for i in (2, 3):
        r = O.phase1_block(q, k, v, i, b, A, theta, scale, rows=[0, b - 1], with_anchor_rows=True)
        np.testing.assert_allclose(r["anchor_out"], first, atol=1e-13)


def test_previous_block_anchor_is_windowed_causal_attention(rng):
    """With the previous block as anchor (the paper's ablation), a row of block
    i >= 2 sees the first A tokens of block i - 1 and causally its own block: a
    windowed causal mask over the true sequence, checked against torch's SDPA.
    Block 1 is plain causal attention and block 2 equals the first-block anchor."""
    L, b, theta, scale = 80, 16, 1e4, 0.3
    q, k, v = _ctx(rng, L, 4, 2, 8)
    pos = np.arange(L)
    qr, kr = O.rope(q, pos, theta), O.rope(k, pos, theta)
    for A in (b, 5):
        prev = O.phase1(q, k, v, b, A, theta, scale, anchor="previous")
        first = O.phase1(q, k, v, b, A, theta, scale)
        np.testing.assert_allclose(prev["out"][1], first["out"][1], atol=1e-13)
        np.testing.assert_allclose(prev["out"][2], first["out"][2], atol=1e-13)
        np.testing.assert_array_equal(prev["k_cache"], first["k_cache"])
        for i in range(1, L // b + 1):
            rows = np.arange((i - 1) * b, i * b)
            keys = pos[None, :]
            vis = (keys <= rows[:, None]) & (keys >= (i - 1) * b)
            if i > 1:
                vis |= (keys >= (i - 2) * b) & (keys < (i - 2) * b + A)
            ro, _ = _torch_sdpa(qr[rows], kr, v, vis, scale)
            np.testing.assert_allclose(prev["out"][i], ro, atol=1e-12)
        # from block 3 on the two anchors differ (otherwise this pin shows nothing)
        assert np.abs(prev["out"][3] - first["out"][3]).max() > 1e-3


def test_anchor_right_before_the_block_is_exact_attention_over_anchor_then_block(rng):
    """Anchor position IDs right before block i, (i-1)b - A .. (i-1)b - 1 (one
    setting of the paper's position ablation): c'_i is then one contiguous run
    of positions and RoPE scores depend only on position differences, so block
    i's rows equal plain causal attention over (first A tokens of c_1, c_i)
    placed at positions 0 .. A + b - 1 (torch's SDPA)."""
    L, b, theta, scale = 80, 16, 1e4, 0.3
    q, k, v = _ctx(rng, L, 4, 2, 8)
    n = L // b
    for A in (b, 5):
        pos = np.array([max((i - 1) * b - A, 0) for i in range(1, n + 1)])
        res = O.phase1(q, k, v, b, A, theta, scale, anchor_pos=pos)
        own = O.phase1(q, k, v, b, A, theta, scale)
        np.testing.assert_array_equal(res["out"][1], own["out"][1])
        np.testing.assert_array_equal(res["k_cache"], own["k_cache"])     # the cache keeps true positions
        p = np.arange(A + b)
        for i in range(2, n + 1):
            tok = np.concatenate([np.arange(A), np.arange((i - 1) * b, i * b)])
            ro, _ = _torch_sdpa(O.rope(q[tok], p, theta), O.rope(k[tok], p, theta), v[tok],
                                np.tril(np.ones((A + b, A + b), dtype=bool)), scale)
            np.testing.assert_allclose(res["out"][i], ro[A:], atol=1e-11)
        # from block 3 on, these positions differ from the anchor's own (else this shows nothing)
        assert np.abs(res["out"][3] - own["out"][3]).max() > 1e-3


def test_anchor_position_ids_only_move_the_anchor(rng):
    """Anchor position IDs drawn from the prefix: all zeros are the anchor's own
    positions; the anchor rows still reproduce block 1's first A rows (they see
    only the anchor, so only differences inside it count); entry i - 1 changes
    block i and no other block."""
    L, b, A, theta, scale = 60, 20, 13, 1e4, 0.3
    q, k, v = _ctx(rng, L, 2, 2, 8)
    own = O.phase1(q, k, v, b, A, theta, scale)
    zero = O.phase1(q, k, v, b, A, theta, scale, anchor_pos=np.zeros(3, dtype=np.int64))
    for i in (1, 2, 3):
        np.testing.assert_array_equal(zero["out"][i], own["out"][i])
    pos = np.array([0, 5, 31])
    res = O.phase1(q, k, v, b, A, theta, scale, anchor_pos=pos)
    for i in (2, 3):
        r = O.phase1_block(q, k, v, i, b, A, theta, scale, rows=[0, b - 1], with_anchor_rows=True, anchor_pos=pos)
        np.testing.assert_allclose(r["anchor_out"], own["out"][1][:A], atol=1e-12)
        assert np.abs(res["out"][i] - own["out"][i]).max() > 1e-3
    moved = O.phase1(q, k, v, b, A, theta, scale, anchor_pos=np.array([0, 5, 2]))
    np.testing.assert_array_equal(moved["out"][2], res["out"][2])
    assert np.abs(moved["out"][3] - res["out"][3]).max() > 1e-3
    np.testing.assert_array_equal(O.augmented_positions(3, b, A, anchor_pos=pos),
                                  np.concatenate([31 + np.arange(A), np.arange(40, 60)]))


def test_phase1_cache_is_rope_of_block_kv(rng):
    L, b, theta = 40, 10, 1e4
    q, k, v = _ctx(rng, L, 2, 1, 8)
    res = O.phase1(q, k, v, b, b, theta, 0.3)
    assert res["k_cache"].shape == (L, 1, 8)                  # L rows: anchor KV discarded
    np.testing.assert_allclose(res["k_cache"], O.rope(k, np.arange(L), theta), atol=1e-13)
    np.testing.assert_array_equal(res["v_cache"], v)
    sub = O.phase1(q, k, v, b, b, theta, 0.3, rows_by_block={i: np.array([0, 3]) for i in range(1, 5)})
    np.testing.assert_allclose(sub["k_cache"], res["k_cache"], atol=1e-13)
    for i in range(1, 5):
        np.testing.assert_allclose(sub["out"][i], res["out"][i][[0, 3]], atol=1e-13)


# ----------------------------------------------------------------------------- merge / Phase 2
def test_merge_is_softmax_over_concatenated_keys(rng):
    q, k, v = _rand(rng, 3, 4, 8), _rand(rng, 30, 2, 8), _rand(rng, 30, 2, 8)
    vis = np.ones((3, 30), dtype=bool)
    cuts = [0, 7, 8, 19, 30]
    parts = [O.attention(q, k[a:c], v[a:c], vis[:, a:c], 0.4) for a, c in zip(cuts, cuts[1:])]
    out, lse = O.merge(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    ro, rl = _torch_sdpa(q, k, v, vis, 0.4)
    np.testing.assert_allclose(out, ro, atol=1e-12)
    np.testing.assert_allclose(lse, rl, atol=1e-12)
    lses = np.stack([p[1] for p in parts])
    np.testing.assert_allclose(lse, logsumexp(lses, axis=0), atol=1e-12)
    w = np.exp(lses - lse[None])
    np.testing.assert_allclose(w.sum(axis=0), 1.0, atol=1e-13)
    # the pages' pairwise update agrees on benign inputs
    po, pl = O.merge_pairwise_literal(np.stack([p[0] for p in parts]), lses)
    np.testing.assert_allclose(po, out, atol=1e-12)
    np.testing.assert_allclose(pl, lse, atol=1e-12)


def test_merge_hazards(rng):
    """Large lse gaps overflow the literal pairwise form; empty partitions get weight 0."""
    o = _rand(rng, 3, 2, 1, 4)
    lse = np.array([[[0.0]], [[800.0]], [[-np.inf]]])
    out, l_ = O.merge(o, lse)
    np.testing.assert_allclose(out, o[1], atol=1e-12)
    np.testing.assert_allclose(l_, 800.0)
    po, _ = O.merge_pairwise_literal(o, lse)
    assert not np.all(np.isfinite(po))                         # the hazard the pages describe
    out, l_ = O.merge(o, np.full((3, 1, 1), -np.inf))
    assert np.all(out == 0) and np.all(l_ == -np.inf)


def _full_sequence(rng, L, T0, S, hq, hkv, d):
    ctx = _ctx(rng, L, hq, hkv, d)
    qry = _ctx(rng, T0, hq, hkv, d)
    dec = _ctx(rng, S, hq, hkv, d)
    return ctx, qry, dec


def test_phase2_equals_global_causal_attention(rng):
    """Query and decode rows after the merge equal exact causal attention over [c, q, generated]."""
    L, b, T0, S, theta, scale = 40, 10, 5, 3, 1e4, 0.3
    (qc, kc, vc), (qq, kq, vq), (qd, kd, vd) = _full_sequence(rng, L, T0, S, 4, 2, 8)
    p1 = O.phase1(qc, kc, vc, b, b, theta, scale)
    Qa, Ka, Va = (np.concatenate(x) for x in ((qc, qq, qd), (kc, kq, kd), (vc, vq, vd)))
    n_all = L + T0 + S
    pos = np.arange(n_all)
    ex, ex_lse = _torch_sdpa(O.rope(Qa, pos, theta), O.rope(Ka, pos, theta), Va,
                             np.tril(np.ones((n_all, n_all), dtype=bool)), scale)
    # query step: T0 rows at positions L.., tail holds their KV
    kt, vt = O.tail_keys(kq, vq, L, theta)
    op, lp = O.phase2_partials(qq, L, p1["k_cache"], p1["v_cache"], b, kt, vt, L, theta, scale)
    assert op.shape[0] == L // b + 1
    out, lse = O.merge(op, lp)
    np.testing.assert_allclose(out, ex[L:L + T0], atol=1e-12)
    np.testing.assert_allclose(lse, ex_lse[L:L + T0], atol=1e-12)
    po, pl = O.phase2_plain(qq, L, p1["k_cache"], p1["v_cache"], kt, vt, L, theta, scale)
    np.testing.assert_allclose(po, out, atol=1e-12)
    np.testing.assert_allclose(pl, lse, atol=1e-12)
    # decode steps: one row each, appended after the query rows
    for s in range(S):
        kt, vt = O.tail_keys(np.concatenate([kq, kd[:s + 1]]), np.concatenate([vq, vd[:s + 1]]), L, theta)
        op, lp = O.phase2_partials(qd[s:s + 1], L + T0 + s, p1["k_cache"], p1["v_cache"], b, kt, vt, L,
                                   theta, scale)
        out, lse = O.merge(op, lp)
        np.testing.assert_allclose(out[0], ex[L + T0 + s], atol=1e-12)
        np.testing.assert_allclose(lse[0], ex_lse[L + T0 + s], atol=1e-12)


def test_phase2_empty_tail_partition(rng):
    L, b, theta, scale = 20, 10, 1e4, 0.3
    (qc, kc, vc), (qq, _, _), _ = _full_sequence(rng, L, 2, 1, 2, 1, 8)
    p1 = O.phase1(qc, kc, vc, b, b, theta, scale)
    empty = np.zeros((0, 1, 8))
    op, lp = O.phase2_partials(qq, L, p1["k_cache"], p1["v_cache"], b, empty, empty, L, theta, scale)
    assert np.all(lp[-1] == -np.inf) and np.all(op[-1] == 0)
    out, lse = O.merge(op, lp)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))


# ----------------------------------------------------------------------------- accounting (host logic)
def test_sizing_matches_pages_arithmetic():
    g = json.load(open(os.path.join(GOLDEN, "sizing.json")))
    c = g["kv_bytes_per_token"]
    per_tok = acc.kv_bytes_per_token(c["n_layers"], c["n_kv_heads"], c["head_dim"], c["elem_bytes"])
    assert per_tok == c["expected"]
    assert per_tok * g["kv_bytes_128k_tokens_GB"]["tokens"] == g["kv_bytes_128k_tokens_GB"]["expected_gib"] * 2 ** 30
    m = g["phase2_message_per_layer_token"]
    assert acc.phase2_message_bytes(m["n_hosts"], m["n_layers"], m["n_tokens"], m["n_heads"], m["head_dim"],
                                    m["elem_bytes"]) == m["expected"]
    t = g["phase2_message_total"]
    tot = acc.phase2_message_bytes(t["n_hosts"], t["n_layers"], t["n_tokens"], t["n_heads"], t["head_dim"],
                                   t["elem_bytes"])
    assert abs(tot / 1e9 - t["expected_gb_approx"]) < 0.005


@pytest.mark.parametrize("anchor", O.ANCHORS)
@pytest.mark.parametrize("L,b,A", [(8, 2, 2), (8, 2, 1), (60, 20, 7), (48, 48, 48), (36, 12, 12)])
def test_phase1_pair_count_brute_force(L, b, A, anchor):
    """Useful pairs = visible (block row, key) pairs of the literal augmented blocks
    (the same count for either anchor block)."""
    count = 0
    for i in range(1, L // b + 1):
        tok, n_anc = O.augmented_block(i, b, A, anchor)
        n = len(tok)
        vis = np.tril(np.ones((n, n), dtype=bool))
        count += int(vis[n_anc:].sum())                          # block rows only
    assert acc.phase1_pairs(L, b, A) == count


def test_phase1_flops_at_workload_sizes():
    w = W.LLAMA8B_128K
    got = [acc.phase1_flops(w.ctx_len, b, b, w.n_q_heads, w.head_dim) for b in (4096, 8192, 16384, 32768)]
    for g_, want in zip(got, (1.29e13, 2.53e13, 4.84e13, 8.80e13)):
        assert abs(g_ / want - 1) < 0.01


def test_phase2_step_bytes_decode_128k():
    w = W.LLAMA8B_128K
    by = acc.phase2_step_bytes(w.ctx_len, w.n_query + 1, 1, w.n_q_heads, w.n_kv_heads, w.head_dim, 2)
    assert abs(by / 2 ** 20 - 512.0) < 0.5                      # 2 * 128K * 8 * 128 * 2 B = 512 MiB


# ----------------------------------------------------------------------------- workloads
def test_bf16_rounding_matches_torch(rng):
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0]            # exact ties
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(W.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workload_generation_is_seeded_and_sinked():
    w = W.SMALL_F32
    a = W.tensor(w, W.T_K_CTX, seed=3)
    b = W.tensor(w, W.T_K_CTX, seed=3)
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, W.tensor(w, W.T_K_CTX, seed=4))
    ws = W.LLAMA8B_32K
    k = W.to_f64(W.tensor(ws.with_block(8192), W.T_K_CTX, seed=0)[:8])
    u = W.sink_direction(ws, 0)
    proj = k @ u                                                   # [8, Hkv]
    assert np.all(proj[:4] > 1.0) and abs(proj[4:].mean()) < 1.0
    assert math.isclose(np.linalg.norm(u), 1.0, rel_tol=1e-12)
