"""GPU parity of libstarattn against the fp64 oracle, through the C ABI.

Small workloads compare every output element (several tiles, ragged tails,
anchor shorter than a block, a single block, GQA groups 1/4/8, head_dim 64 and
128). The five full-size workloads compare a seeded sample of context rows and
every Phase-2 row, in the launch configuration the benchmark uses.
"""
import numpy as np
import pytest
import torch

import workloads as W
from harness import assert_close, check_workload, log, run_oracle, to_device, to_host
import long_context_attention_amd as sa
from long_context_attention_amd.runner import StarLayer

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    sa._binding.lib()


SMALL = [
    W.SMALL_F32,
    # ragged blocks (b not a multiple of any tile), anchor shorter than a block
    W.Workload("ragged_f32", 101, "f32", 2, 1, 64, 600, 200, 136, 5, 3, 1.0e4, False),
    W.Workload("ragged_bf16", 102, "bf16", 8, 2, 128, 3 * 328, 328, 200, 7, 3, 5.0e5, True),
    # a single block: Phase 1 is plain causal attention
    W.Workload("single_block_bf16", 103, "bf16", 4, 4, 128, 384, 384, 384, 3, 2, 1.0e4, False),
    # GQA group of 8, head_dim 64
    W.Workload("gqa8_d64_bf16", 104, "bf16", 16, 2, 64, 4 * 256, 256, 256, 9, 2, 1.0e4, True),
    # blocks shorter than one key tile, many blocks, anchor of 17 tokens
    W.Workload("tiny_blocks_bf16", 105, "bf16", 4, 1, 128, 8 * 40, 40, 17, 4, 4, 1.0e4, False),
    # float32 at head_dim 128, anchor of one token
    W.Workload("f32_d128_a1", 106, "f32", 4, 2, 128, 2 * 160, 160, 1, 4, 2, 1.0e4, False),
    # query step of 40 tokens x 8 heads = 320 rows per KV head: two row tiles, the second ragged
    W.Workload("multi_tile_query_bf16", 110, "bf16", 32, 4, 128, 2 * 512, 512, 512, 40, 2, 5.0e5, True),
    # query step of 600 tokens (10 row tiles per KV head): a tail longer than 8 key tiles is a
    # partition with tile-kernel workgroups of its own (3 chunks, the last ragged), not folded
    W.Workload("long_query_bf16", 143, "bf16", 8, 2, 128, 2 * 512, 512, 512, 600, 2, 1.0e4, True),
    # multi-head attention (group of 1) through the tile kernel: 40 query rows per KV head
    W.Workload("mha_query_bf16", 144, "bf16", 4, 4, 128, 2 * 256, 256, 256, 40, 2, 1.0e4, False),
    # head_dim 64, group of 8, a query step over two row tiles per KV head (320 rows)
    W.Workload("d64_two_tile_query_bf16", 145, "bf16", 16, 2, 64, 2 * 256, 256, 256, 40, 2, 1.0e4, True),
    # query step of 2 tokens x 4 heads = 8 rows: the streaming decode kernel with two tokens
    # (causal between them in the tail), head_dim 64, anchor shorter than a block
    W.Workload("two_token_query_bf16", 111, "bf16", 8, 2, 64, 3 * 192, 192, 96, 2, 3, 1.0e4, True),
    # the previous block as anchor (the paper's ablation): fp32, and bf16 with ragged blocks and A < b
    W.SMALL_F32.with_anchor("previous"),
    W.Workload("prev_anchor_ragged_bf16", 113, "bf16", 8, 2, 128, 4 * 328, 328, 200, 7, 3, 5.0e5, True, "previous"),
    # the anchor at other position IDs (the paper's position ablation): random ones from the
    # prefix and the ones right before the block; fp32, ragged bf16 with A < b, tiny blocks
    W.SMALL_F32.with_anchor_at("random"),
    W.SMALL_F32.with_anchor_at("adjacent"),
    W.Workload("anchor_at_ragged_bf16", 114, "bf16", 8, 2, 128, 4 * 328, 328, 200, 7, 3, 5.0e5, True,
               anchor_at="random"),
    W.Workload("anchor_at_tiny_bf16", 115, "bf16", 4, 1, 128, 8 * 40, 40, 17, 4, 4, 1.0e4, False,
               anchor_at="random"),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_workloads_full_parity(w):
    check_workload(w, seed=0, full_rows=True)


FULL = [W.LLAMA8B_32K.with_block(8192), *W.LLAMA8B_128K_SWEEP, W.LLAMA70B_128K.with_block(32768),
        W.LLAMA8B_1M.with_block(65536), W.LLAMA8B_128K.with_block(4096).with_anchor("previous"),
        W.LLAMA8B_128K.with_block(32768).with_anchor("previous"),
        W.LLAMA8B_128K.with_block(4096).with_anchor_at("random"),
        W.LLAMA8B_128K.with_block(32768).with_anchor_at("adjacent")]


def row_tile_tokens(w) -> int:
    """Tokens per Phase-1 row tile: 256 rows of the largest power of two (<= 8)
    of query heads dividing the GQA group."""
    gp = 1
    while gp < 8 and w.group % (2 * gp) == 0:
        gp *= 2
    return 256 // gp


# Workloads whose sample holds one random row in every Phase-1 row tile of every
# block (several full super-rounds of 32 row tiles per block).
EVERY_TILE = ("llama8b_32k@b8192", "llama8b_128k@b32768")


@pytest.mark.parametrize("w", FULL, ids=[w.name for w in FULL])
def test_full_size_workloads_sampled_parity(w):
    rows = W.sample_rows(w, 0, span=row_tile_tokens(w)) if w.name in EVERY_TILE else None
    if rows is not None:
        log(f"{w.name}: {sum(len(r) for r in rows.values())} context rows, every row tile of every block")
    check_workload(w, seed=0, full_rows=False, rows_by_block=rows)


FUSED = [w for w in SMALL if w.name in ("small_f32_2k", "ragged_bf16", "tiny_blocks_bf16", "multi_tile_query_bf16",
                                         "two_token_query_bf16", "gqa8_d64_bf16", "long_query_bf16")] + [
    # a query step with one row tile per KV head, the tail riding with a
    # context chunk of 4 key tiles
    W.Workload("fold_query_bf16", 142, "bf16", 8, 2, 128, 4 * 512, 512, 512, 40, 2, 1.0e4, True),
    W.LLAMA8B_128K.with_block(32768)]


@pytest.mark.parametrize("w", FUSED, ids=[w.name for w in FUSED])
def test_fused_step_matches_oracle(w):
    """sa_phase2_step (append, partials, every chunk merged straight into the
    output) for the query step and every decode step, against the oracle's
    merged output and LSE."""
    x = W.all_tensors(w, 0)
    d = {k: to_device(v) for k, v in x.items()}
    layer = StarLayer.for_workload(w)
    layer.encode(d["q_ctx"], d["k_ctx"], d["v_ctx"])
    for t in (layer.k_tail, layer.v_tail):
        t.fill_(float("nan"))                # rows the steps do not write stay NaN and must not be read
    log(f"{w.name}: fused steps")
    got = [[to_host(t) for t in layer.step_fused(d["q_qry"], d["k_qry"], d["v_qry"])]]
    for s in range(w.n_decode):
        got.append([to_host(t) for t in layer.step_fused(d["q_dec"][s:s + 1], d["k_dec"][s:s + 1],
                                                          d["v_dec"][s:s + 1])])
    torch.cuda.synchronize()
    n_new = w.n_query + w.n_decode
    tails = to_host(layer.k_tail[:, :n_new]), to_host(layer.v_tail[:, :n_new])
    del layer, d
    ref = run_oracle(w, x, {i: np.array([0]) for i in range(1, w.n_blocks + 1)}, np.array([0]))
    want = [(ref["qry"]["out"], ref["qry"]["lse"])] + [(r["out"], r["lse"]) for r in ref["dec"]]
    for i, ((go, gl), (wo, wl)) in enumerate(zip(got, want)):
        assert_close(f"{w.name} fused step {i} out", go, wo, w.dtype)
        assert_close(f"{w.name} fused step {i} lse", gl, wl, w.dtype)
    # the rows the steps appended (the decode kernel writes them itself in decode-shaped steps)
    assert_close(f"{w.name} fused k_tail", tails[0], ref["k_tail"], w.dtype)
    assert_close(f"{w.name} fused v_tail", tails[1], ref["v_tail"], w.dtype)


# A batch of sequences with different context and block lengths (and anchors),
# and a batch of three 32K sequences with different inputs.
BATCH_SMALL = [W.Workload("batch_a", 120, "bf16", 8, 2, 128, 4 * 256, 256, 256, 4, 3, 5.0e5, True),
               W.Workload("batch_b", 121, "bf16", 8, 2, 128, 3 * 512, 512, 512, 7, 3, 5.0e5, True),
               W.Workload("batch_c", 122, "bf16", 8, 2, 128, 2 * 320, 320, 200, 1, 3, 5.0e5, True)]
BATCH_32K = [(W.LLAMA8B_32K, 0), (W.LLAMA8B_32K, 1), (W.LLAMA8B_32K, 2)]
# 8 query heads per KV head at head_dim 64 (the other decode-kernel variant), A < b
BATCH_G8_D64 = [W.Workload("batch_d", 123, "bf16", 16, 2, 64, 2 * 256, 256, 256, 2, 3, 1.0e4, True),
                W.Workload("batch_e", 124, "bf16", 16, 2, 64, 3 * 128, 128, 64, 3, 3, 1.0e4, True)]


@pytest.mark.parametrize("batch", [[(w, 0) for w in BATCH_SMALL], BATCH_32K, [(w, 0) for w in BATCH_G8_D64]],
                         ids=["mixed_small", "three_32k", "g8_d64"])
def test_batched_decode_matches_oracle(batch):
    """sa_decode_step_batched over sequences of different lengths, each after its
    own query step, against the oracle's decode outputs of each sequence."""
    layers, devs, hosts = [], [], []
    for w, seed in batch:
        x = W.all_tensors(w, seed)
        d = {k: to_device(v) for k, v in x.items()}
        layer = StarLayer.for_workload(w)
        layer.encode(d["q_ctx"], d["k_ctx"], d["v_ctx"])
        for t in (layer.k_tail, layer.v_tail):
            t.fill_(float("nan"))            # rows no step writes stay NaN and must not be read
        layer.step(d["q_qry"], d["k_qry"], d["v_qry"])
        layers.append(layer), devs.append(d), hosts.append(x)
    w0 = batch[0][0]
    outs = [torch.empty(w0.n_q_heads, w0.head_dim, device="cuda", dtype=torch.bfloat16) for _ in batch]
    lses = [torch.empty(w0.n_q_heads, device="cuda") for _ in batch]
    got = []
    for s in range(min(w.n_decode for w, _ in batch)):
        seqs = [dict(q=d["q_dec"][s], k_new=d["k_dec"][s], v_new=d["v_dec"][s], k_cache=l.k_cache, v_cache=l.v_cache,
                     k_tail=l.k_tail, v_tail=l.v_tail, out=o, lse=ls, ctx_len=l.L, block_len=l.b, tail_cap=l.tail_cap,
                     tail_len=l.tail_len) for d, l, o, ls in zip(devs, layers, outs, lses)]
        ws = torch.empty(sa.sa_decode_batch_workspace_bytes(layers[0].desc, seqs), dtype=torch.uint8, device="cuda")
        sa.sa_decode_step_batched(layers[0].desc, seqs, ws)
        torch.cuda.synchronize()
        for l in layers:
            l.tail_len += 1
        got.append([(to_host(o), to_host(ls)) for o, ls in zip(outs, lses)])
    tails = [(to_host(l.k_tail[:, :l.tail_len]), to_host(l.v_tail[:, :l.tail_len])) for l in layers]
    del layers, devs
    for i, ((w, seed), x) in enumerate(zip(batch, hosts)):
        log(f"batched decode: oracle of sequence {i} ({w.name}, seed {seed})")
        ref = run_oracle(w, x, {j: np.array([0]) for j in range(1, w.n_blocks + 1)}, np.array([0]))
        for s, step in enumerate(got):
            assert_close(f"batch seq {i} step {s} out", step[i][0], ref["dec"][s]["out"][0], w.dtype)
            assert_close(f"batch seq {i} step {s} lse", step[i][1], ref["dec"][s]["lse"][0], w.dtype)
        # the query step's rows and the rows the batched kernel appended itself
        n = tails[i][0].shape[1]
        assert_close(f"batch seq {i} k_tail", tails[i][0], ref["k_tail"][:, :n], w.dtype)
        assert_close(f"batch seq {i} v_tail", tails[i][1], ref["v_tail"][:, :n], w.dtype)


@pytest.mark.parametrize("w", [W.Workload("zero_pos_bf16", 116, "bf16", 8, 2, 128, 4 * 200, 200, 136, 3, 1, 5.0e5,
                                           True),
                               W.Workload("zero_pos_f32", 117, "f32", 4, 1, 64, 3 * 96, 96, 96, 3, 1, 1.0e4, False)],
                         ids=["bf16", "f32"])
def test_anchor_at_zero_positions_is_encode_bit_for_bit(w):
    """All-zero anchor positions are the anchor's own: the rotated anchor keys in
    the workspace then equal the cache's first rows, so the workspace kernel
    must reproduce sa_phase1_encode exactly (and keep the same cache)."""
    x = {k: to_device(v) for k, v in W.all_tensors(w, 0).items()}
    ref = StarLayer.for_workload(w)
    ref.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
    at = StarLayer.for_workload(w, anchor_pos=[0] * w.n_blocks)
    at.anchor_ws.fill_(7)                                   # stale workspace contents must not matter
    at.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
    torch.cuda.synchronize()
    for name in ("out_ctx", "k_cache", "v_cache"):
        assert torch.equal(getattr(at, name), getattr(ref, name)), name


def test_repeat_calls_are_bitwise_deterministic():
    w = W.Workload("det_bf16", 107, "bf16", 8, 2, 128, 4 * 256, 256, 256, 5, 2, 5.0e5, True)
    x = {k: to_device(v) for k, v in W.all_tensors(w, 1).items()}
    outs = []
    for _ in range(2):
        layer = StarLayer.for_workload(w)
        layer.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
        o, l_, _, _ = layer.step(x["q_qry"], x["k_qry"], x["v_qry"])
        o2, l2, _, _ = layer.step(x["q_dec"][:1], x["k_dec"][:1], x["v_dec"][:1])
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (layer.out_ctx, layer.k_cache, layer.v_cache, o, l_, o2, l2)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_decode_partials_do_not_depend_on_workspace_contents():
    """Whatever the Phase-2 workspace holds before a decode step (zeros, random
    bytes, what an earlier call left, all ones), the partials and the merged
    output are the same, bit for bit: the workspace is scratch only."""
    w = W.Workload("ws_bf16", 109, "bf16", 8, 2, 128, 3 * 512, 512, 512, 4, 3, 5.0e5, True)
    x = {k: to_device(v) for k, v in W.all_tensors(w, 2).items()}
    layer = StarLayer.for_workload(w)
    layer.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
    layer.step(x["q_qry"], x["k_qry"], x["v_qry"])
    ws = layer.workspace
    gen = torch.Generator(device="cuda").manual_seed(5)
    results = []
    for fill in ("zeros", "random", "previous", "ones"):
        layer.tail_len = w.n_query        # replay the same first decode step
        if fill == "zeros":
            ws.zero_()
        elif fill == "random":
            ws.copy_(torch.randint(0, 256, ws.shape, generator=gen, device="cuda", dtype=torch.uint8))
        elif fill == "ones":
            ws.fill_(255)
        o, l_, op, lp = layer.step(x["q_dec"][:1], x["k_dec"][:1], x["v_dec"][:1])
        torch.cuda.synchronize()
        results.append([t.clone() for t in (o, l_, op, lp)])
    for other in results[1:]:
        for a, b in zip(results[0], other):
            assert torch.equal(a, b)


def test_two_streams_match_one_after_the_other():
    """Two layers' Phase 1 and steps (sa_phase2_step), launched alternately on two
    streams so that they run at once, give bit for bit what the same calls give
    one after the other on one stream: no call keeps state for another."""
    w = W.Workload("streams_bf16", 146, "bf16", 8, 2, 128, 4 * 512, 512, 512, 40, 2, 1.0e4, True)
    xs = [{k: to_device(v) for k, v in W.all_tensors(w, seed).items()} for seed in (0, 1)]

    main = torch.cuda.current_stream()

    def run(streams):
        layers = [StarLayer.for_workload(w) for _ in xs]
        for s in streams:
            s.wait_stream(main)                   # inputs and the layers' buffers were made on this stream
        got = [[] for _ in xs]
        n_calls = 2 + w.n_decode
        for i in range(n_calls):
            for j, (layer, x) in enumerate(zip(layers, xs)):
                s = streams[j]
                with torch.cuda.stream(s):
                    if i == 0:
                        layer.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"], s)
                        got[j] += [layer.out_ctx.clone(), layer.k_cache.clone(), layer.v_cache.clone()]
                    elif i == 1:
                        got[j] += [t.clone() for t in layer.step_fused(x["q_qry"], x["k_qry"], x["v_qry"], s)]
                    else:
                        d = i - 2
                        got[j] += [t.clone() for t in layer.step_fused(x["q_dec"][d:d + 1], x["k_dec"][d:d + 1],
                                                                        x["v_dec"][d:d + 1], s)]
        for j, layer in enumerate(layers):
            with torch.cuda.stream(streams[j]):
                got[j] += [layer.k_tail.clone(), layer.v_tail.clone()]
        torch.cuda.synchronize()
        return got

    ref = run([main, main])
    got = run([torch.cuda.Stream(), torch.cuda.Stream()])
    for j in range(len(xs)):
        for k, (a, b) in enumerate(zip(got[j], ref[j])):
            assert torch.equal(a, b), f"layer {j}, tensor {k}"


def test_decode_step_replays_in_a_hip_graph():
    """A decode step (append, partials, merge) captured once in a HIP graph and
    replayed several times, with eager work and synchronisation in between,
    reproduces the eager step bit for bit on every replay."""
    w = W.Workload("graph_bf16", 110, "bf16", 8, 2, 128, 4 * 256, 256, 256, 4, 2, 5.0e5, True)
    x = {k: to_device(v) for k, v in W.all_tensors(w, 3).items()}
    layer = StarLayer.for_workload(w)
    layer.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
    layer.step(x["q_qry"], x["k_qry"], x["v_qry"])
    q, k, v = (x[n][:1].clone() for n in ("q_dec", "k_dec", "v_dec"))
    layer.tail_len = w.n_query
    ref = [t.clone() for t in layer.step(q, k, v)]
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer.tail_len = w.n_query
        with torch.cuda.graph(graph, stream=side):
            outs = layer.step(q, k, v)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan")) if t.is_floating_point() else t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, outs):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        scratch.mul_(1.0001).add_(rep)          # unrelated eager work between replays
        layer.workspace.random_()               # and a scrambled workspace
        torch.cuda.synchronize()


def _replay_matches(capture, outs_ref, scramble):
    """Capture `capture()` once in a HIP graph, replay it four times with eager
    work, a scrambled workspace and NaN-filled outputs in between, and check
    every replay against the eager outputs bit for bit."""
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            outs = capture()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(outs_ref, outs):
            assert torch.equal(a, b), f"replay {rep} differs from the eager call"
        junk.mul_(1.0001).add_(rep)
        scramble()
        torch.cuda.synchronize()


def test_fused_and_batched_steps_replay_in_a_hip_graph():
    """sa_phase2_step and sa_decode_step_batched captured in HIP graphs replay
    bit for bit (each replay rewrites the same tail row with the same values)."""
    w = W.Workload("graph2_bf16", 125, "bf16", 8, 2, 128, 4 * 256, 256, 256, 4, 2, 5.0e5, True)
    x = {k: to_device(v) for k, v in W.all_tensors(w, 4).items()}
    layers = []
    for _ in range(2):
        l_ = StarLayer.for_workload(w)
        l_.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
        l_.step(x["q_qry"], x["k_qry"], x["v_qry"])
        layers.append(l_)
    q, k, v = (x[n][:1].clone() for n in ("q_dec", "k_dec", "v_dec"))
    l0 = layers[0]

    def fused():
        l0.tail_len = w.n_query
        return [t for t in l0.step_fused(q, k, v)]
    ref = [t.clone() for t in fused()]
    torch.cuda.synchronize()
    _replay_matches(fused, ref, lambda: l0.workspace.random_())

    outs = [torch.empty(w.n_q_heads, w.head_dim, device="cuda", dtype=torch.bfloat16) for _ in layers]
    lses = [torch.empty(w.n_q_heads, device="cuda") for _ in layers]
    seqs = sa.decode_seqs([dict(q=q[0], k_new=k[0], v_new=v[0], k_cache=l_.k_cache, v_cache=l_.v_cache,
                                k_tail=l_.k_tail, v_tail=l_.v_tail, out=o, lse=ls, ctx_len=l_.L, block_len=l_.b,
                                tail_cap=l_.tail_cap, tail_len=w.n_query)
                           for l_, o, ls in zip(layers, outs, lses)])
    ws = torch.empty(sa.sa_decode_batch_workspace_bytes(l0.desc, seqs), dtype=torch.uint8, device="cuda")

    def batched():
        sa.sa_decode_step_batched(l0.desc, seqs, ws)
        return outs + lses
    ref = [t.clone() for t in batched()]
    torch.cuda.synchronize()
    # the batched step of sequence 0 equals its fused step (same inputs) to rounding
    assert_close("batched vs fused out", to_host(ref[0]), to_host(fused()[0][0]), "bf16")
    _replay_matches(batched, ref, lambda: ws.random_())


def test_empty_tail_partition_and_noop_append():
    """A partition without visible keys returns lse = -inf and weight 0 (never NaN)."""
    w = W.Workload("empty_tail", 108, "bf16", 4, 1, 128, 2 * 128, 128, 128, 2, 1, 1.0e4, False)
    x = {k: to_device(v) for k, v in W.all_tensors(w, 0).items()}
    layer = StarLayer.for_workload(w)
    layer.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
    sa.sa_decode_append(layer.desc, None, None, 0, w.ctx_len, layer.k_tail, layer.v_tail, layer.tail_cap, 0)
    t = w.n_query
    op = torch.empty(layer.n_parts, t, w.n_q_heads, w.head_dim, device="cuda")
    lp = torch.empty(layer.n_parts, t, w.n_q_heads, device="cuda")
    sa.sa_phase2_partial(layer.desc, x["q_qry"], t, w.ctx_len, layer.k_cache, layer.v_cache, w.ctx_len, w.block_len,
                         layer.k_tail, layer.v_tail, layer.tail_cap, 0, w.ctx_len, op, lp, layer.workspace)
    out = torch.empty(t, w.n_q_heads, w.head_dim, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(t, w.n_q_heads, device="cuda")
    sa.sa_phase2_merge(layer.n_parts, t, w.n_q_heads, w.head_dim, op, lp, out, sa.SA_BF16, lse)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(lp[-1])) and torch.all(op[-1] == 0)
    assert torch.all(torch.isfinite(lse)) and torch.all(torch.isfinite(out.float()))
    # merging only empty partitions gives out 0 and lse -inf
    sa.sa_phase2_merge(1, t, w.n_q_heads, w.head_dim, op[-1:].contiguous(), lp[-1:].contiguous(), out, sa.SA_BF16,
                       lse)
    torch.cuda.synchronize()
    assert torch.all(torch.isneginf(lse)) and torch.all(out.float() == 0)


def test_absent_tail_buffer_matches_empty_tail():
    """tail_cap 0 with no tail buffers (null pointers) on the decode kernel gives
    the same partials, bit for bit, as an allocated but empty tail."""
    w = W.Workload("no_tail", 112, "bf16", 8, 2, 128, 2 * 256, 256, 256, 1, 1, 1.0e4, False)
    x = {k: to_device(v) for k, v in W.all_tensors(w, 0).items()}
    layer = StarLayer.for_workload(w)
    layer.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
    t = 1
    res = []
    for k_tail, v_tail, cap in ((layer.k_tail, layer.v_tail, layer.tail_cap), (None, None, 0)):
        op = torch.empty(layer.n_parts, t, w.n_q_heads, w.head_dim, device="cuda")
        lp = torch.empty(layer.n_parts, t, w.n_q_heads, device="cuda")
        sa.sa_phase2_partial(layer.desc, x["q_qry"][:t], t, w.ctx_len, layer.k_cache, layer.v_cache, w.ctx_len,
                             w.block_len, k_tail, v_tail, cap, 0, w.ctx_len, op, lp, layer.workspace)
        torch.cuda.synchronize()
        res.append((op, lp))
    assert torch.all(torch.isneginf(res[1][1][-1])) and torch.all(res[1][0][-1] == 0)
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_workspace_too_small_is_rejected_on_device_buffers():
    w = W.SMALL_F32
    layer = StarLayer.for_workload(w)
    small = torch.empty(64, dtype=torch.uint8, device="cuda")
    q = torch.zeros(w.n_query, w.n_q_heads, w.head_dim, device="cuda")
    with pytest.raises(sa.StarAttnError) as e:
        sa.sa_phase2_partial(layer.desc, q, w.n_query, w.ctx_len, layer.k_cache, layer.v_cache, w.ctx_len,
                             w.block_len, layer.k_tail, layer.v_tail, layer.tail_cap, 0, w.ctx_len,
                             layer._out_part, layer._lse_part, small)
    assert e.value.code == sa.SA_EWORKSPACE


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_queries_inside_the_context_mask_later_keys(dtype):
    """sa_phase2_partial with queries at positions inside the context (keys past a
    query's position are invisible in every partition): 1 and 2 tokens (the
    streaming decode kernel's two row counts for bf16), 3 tokens (the tile
    kernel for bf16) and the float32 kernel, at positions inside block 1, in the
    middle of block 2, on a block boundary and at the last context position,
    against the oracle's partials."""
    import oracle as O
    w = W.Workload(f"ctx_queries_{dtype}", 133, dtype, 8, 2, 128, 4 * 512, 512, 512, 3, 1, 1.0e4, True)
    xh = W.all_tensors(w, 0)
    x = {k: to_device(v) for k, v in xh.items()}
    layer = StarLayer.for_workload(w, max_t_q=3)
    layer.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
    torch.cuda.synchronize()
    f = {k: W.to_f64(v) for k, v in xh.items()}
    kc = O.rope(f["k_ctx"], np.arange(w.ctx_len), w.rope_theta)
    vc = f["v_ctx"]
    empty = np.zeros((0, w.n_kv_heads, w.head_dim))
    for t in (1, 2, 3):
        ws = torch.empty(sa.sa_workspace_bytes(sa.SA_CALL_PHASE2, layer.desc, w.ctx_len, w.block_len, t,
                                               layer.tail_cap), dtype=torch.uint8, device="cuda")
        for pos in (3, 700, 1024, w.ctx_len - 1):
            op = torch.empty(layer.n_parts, t, w.n_q_heads, w.head_dim, device="cuda")
            lp = torch.empty(layer.n_parts, t, w.n_q_heads, device="cuda")
            sa.sa_phase2_partial(layer.desc, x["q_qry"][:t], t, pos, layer.k_cache, layer.v_cache, w.ctx_len,
                                 w.block_len, layer.k_tail, layer.v_tail, layer.tail_cap, 0, w.ctx_len, op, lp, ws)
            torch.cuda.synchronize()
            want_o, want_l = O.phase2_partials(f["q_qry"][:t], pos, kc, vc, w.block_len, empty, empty, w.ctx_len,
                                               w.rope_theta, w.softmax_scale)
            log(f"context queries: t={t} pos={pos}")
            assert_close(f"t={t} pos={pos} lse_part", to_host(lp), want_l, w.dtype)
            assert_close(f"t={t} pos={pos} out_part", to_host(op), want_o, w.dtype)


def _wide_range_inputs(w: W.Workload, x: dict, seed: int) -> tuple[dict, dict]:
    """Multiply the keys by factors from 1/4 to 14: per group of 64 context
    positions a staircase, rising over groups 0-7 and falling over groups
    8-15 (repeating), so that a row's key-tile maxima span about 57 in log2
    units (neighbouring tiles differ by 6.5 at the median, up to 52) and the
    running softmax reference falls behind by more than the 2^32 bound on a
    tile's row sum and must move, in both directions; the query and decode
    keys get seeded random factors from the same set.

    bf16 operands carry score errors in proportion to the scores' scale
    (about 0.01 natural-log units here), and an output error is such an error
    times the spread of the values it weighs; the values are divided by 16
    for bf16 (exactly), which keeps correct arithmetic at about half the
    tolerance while a reference move that loses, skips or misweighs the rows'
    earlier sum still misses it by several times. Inputs are rounded to the
    workload's type once, and both sides get them. Returns the inputs and the
    key factors per context row and per tail row."""
    steps = np.array([0.25, 2.0, 4.0, 6.0, 8.0, 10.0, 12.0, 14.0], dtype=np.float32)
    g = np.arange((w.ctx_len + 63) // 64)
    groups = np.where((g // 8) % 2 == 0, steps[g % 8], steps[7 - g % 8])
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, w.config_id, 2000])))
    fac = {"k_ctx": np.repeat(groups, 64)[:w.ctx_len],
           "k_qry": rng.choice(steps, size=w.n_query), "k_dec": rng.choice(steps, size=w.n_decode)}
    if w.dtype == "bf16":
        for name in ("v_ctx", "v_qry", "v_dec"):
            fac[name] = np.full(x[name].shape[0], 1.0 / 16, dtype=np.float32)
    out = dict(x)
    for name, f in fac.items():
        v = x[name]
        vf = (W.bf16_bits_to_f32(v) if v.dtype == np.uint16 else v) * f[:, None, None]
        out[name] = W.f32_to_bf16_bits(vf) if v.dtype == np.uint16 else vf.astype(np.float32)
    return out, {"k_ctx": fac["k_ctx"], "k_tail": np.concatenate([fac["k_qry"], fac["k_dec"]])}


@pytest.mark.parametrize("w", [W.Workload("wide_range_bf16", 140, "bf16", 8, 2, 128, 4 * 512, 512, 512, 40, 3, 1.0e4,
                                          True),
                               W.Workload("wide_range_f32", 141, "f32", 8, 2, 128, 3 * 320, 320, 200, 40, 3, 1.0e4,
                                          True)], ids=["bf16", "f32"])
def test_wide_score_range_across_key_tiles(w):
    """Scores whose scale jumps between key tiles (the running softmax reference
    must move by many powers of two, and a tile far below it must vanish without
    harm): Phase 1, the query step and decode steps, every element against the
    oracle on the same scaled inputs."""
    import oracle as O
    x, key_scale = _wide_range_inputs(w, W.all_tensors(w, 0), 0)
    lse_tol = None
    if w.dtype == "bf16":
        # A log-sum-exp moves by at most the largest error of one of its scores.
        # Rounding the rotated query and key to bf16 (2^-9 relative each) and
        # float32 accumulation bound a score's error by (2^-8 + 2^-16) times
        # sum_i |q_i k_i| times the softmax scale; the bound is taken over every
        # Phase-2 query row and key, added to the standard allowance.
        n_new = w.n_query + w.n_decode
        pos_new = w.ctx_len + np.arange(n_new)
        q = O.rope(W.to_f64(np.concatenate([x["q_qry"], x["q_dec"]])), pos_new, w.rope_theta)
        k = np.concatenate([O.rope(W.to_f64(x["k_ctx"]), np.arange(w.ctx_len), w.rope_theta),
                            O.rope(W.to_f64(np.concatenate([x["k_qry"], x["k_dec"]])), pos_new, w.rope_theta)])
        worst = max(float((np.abs(q[:, h]) @ np.abs(k[:, h // w.group]).T).max()) for h in range(w.n_q_heads))
        lse_tol = 2e-2 + (2.0 ** -8 + 2.0 ** -16) * worst * w.softmax_scale
        log(f"{w.name}: log-sum-exp tolerance {lse_tol:.3f}")
    check_workload(w, seed=0, full_rows=True, x=x, key_scale=key_scale, lse_tol=lse_tol)


@pytest.mark.parametrize("w", [W.Workload("order_ragged_bf16", 134, "bf16", 8, 2, 128, 3 * 328, 328, 200, 2, 1, 5.0e5,
                                          True), W.LLAMA8B_32K.with_block(8192)], ids=["ragged", "llama8b_32k"])
def test_phase1_job_order_does_not_change_results(w):
    """Phase 1 with the run-time job order (a workspace for its counters) and
    with the static order (no workspace) gives the same outputs and caches, bit
    for bit, twice in a row (the counters are reset by every call)."""
    x = {k: to_device(v) for k, v in W.all_tensors(w, 0).items()}
    ref = StarLayer.for_workload(w)
    sa.sa_phase1_encode(ref.desc, w.ctx_len, w.block_len, w.anchor_len, x["q_ctx"], x["k_ctx"], x["v_ctx"],
                        ref.out_ctx, ref.k_cache, ref.v_cache, None)
    dyn = StarLayer.for_workload(w)
    for rep in range(2):
        dyn.out_ctx.fill_(float("nan"))
        dyn.p1_ws.fill_(0xAB if rep else 0)      # stale counters must not matter
        dyn.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
        torch.cuda.synchronize()
        for name in ("out_ctx", "k_cache", "v_cache"):
            assert torch.equal(getattr(dyn, name), getattr(ref, name)), f"{name}, call {rep}"
