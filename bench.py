#!/usr/bin/env python3
"""Star Attention hot-path benchmark on one MI355X.

One step = the whole hot path over one synthetic layer: Phase 1 (RoPE + KV
cache + anchor-augmented blockwise attention over the context), the query step
(append, local attention of every partition, global merge) and every decode
step. Default workload: Llama-3.1-8B-shaped layer at 128K context
(32 query heads, 8 KV heads, head_dim 128, bf16, b = 32768 = L/4).

Headline ``value``: Phase-1 useful TFLOP/s (anchor rows and masked pairs not
counted). ``phase2``: decode GB/s (visible KV + query + output bytes per step,
over the partial + merge time, with the caches evicted from L2/MALL before
each timed step). Times come from HIP events on the stream the library
launches on. ``star_vs_global`` runs the same Phase-1 kernel with one block
(exact causal attention over the whole context) and reports the time ratio and
the deviation of Star Attention's context outputs from it (context only), and
the same for the paper's anchor ablation (the previous block as anchor).
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as W  # noqa: E402
from long_context_attention_amd import accounting as acc  # noqa: E402

METRIC = "Phase-1 anchor-block attn TFLOP/s; Phase-2 global-attn GB/s at 128K ctx"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def to_device(arr: np.ndarray):
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(arr).to("cuda")


def run_steps(layer, x, w, n_steps: int, record: bool):
    """Run n_steps whole hot-path steps; returns per-step event timings (ms) if record."""
    import torch
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    rec = []
    for _ in range(n_steps):
        e = {"p1": (ev(), ev()), "q": (ev(), ev(), ev()), "d": [(ev(), ev(), ev()) for _ in range(w.n_decode)]}
        e["p1"][0].record()
        layer.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
        e["p1"][1].record()
        e["q"][0].record()
        layer.step(x["q_qry"], x["k_qry"], x["v_qry"])
        e["q"][2].record()
        for s in range(w.n_decode):
            a, b_, c = e["d"][s]
            a.record()
            layer.step(x["q_dec"][s:s + 1], x["k_dec"][s:s + 1], x["v_dec"][s:s + 1])
            c.record()
        rec.append(e)
    torch.cuda.synchronize()
    if not record:
        return None
    out = []
    for e in rec:
        out.append({"p1": e["p1"][0].elapsed_time(e["p1"][1]),
                    "q": e["q"][0].elapsed_time(e["q"][2]),
                    "d": [a.elapsed_time(c) for a, _, c in e["d"]]})
    return out


def phase2_only(layer, x, w, reps: int, flush=None):
    """Decode-step partial + merge timing (ms) with the tail already holding T0 + s rows."""
    import torch
    from long_context_attention_amd import _binding as B
    t = 1
    times = []
    n = layer.n_parts * t * layer.hq
    op = layer._out_part[: n * layer.d].view(layer.n_parts, t, layer.hq, layer.d)
    lp = layer._lse_part[:n].view(layer.n_parts, t, layer.hq)
    q = x["q_dec"][:1]
    tail_len = w.n_query + 1
    for _ in range(reps):
        if flush is not None:
            flush.sum()   # read-only sweep: evicts the cached KV without leaving dirty lines behind
        a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        B.sa_phase2_partial(layer.desc, q, t, w.ctx_len + w.n_query, layer.k_cache, layer.v_cache, w.ctx_len,
                            w.block_len, layer.k_tail, layer.v_tail, layer.tail_cap, tail_len, w.ctx_len, op, lp,
                            layer.workspace)
        B.sa_phase2_merge(layer.n_parts, t, layer.hq, layer.d, op, lp, layer.out[:t], layer.dtype, layer.lse[:t])
        c.record()
        times.append((a, c))
    torch.cuda.synchronize()
    return [a.elapsed_time(c) for a, c in times]


def rope_cache_ms(layer, x, w, reps: int = 5) -> float:
    """Median time (ms) of Phase 1's RoPE/cache kernel alone: the same kernel with
    the same sizes and arguments, launched through sa_decode_append over every
    context row into the layer's own cache (rewriting the values Phase 1 wrote)."""
    import torch
    from long_context_attention_amd import _binding as B
    ts = []
    for _ in range(reps + 1):
        a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        B.sa_decode_append(layer.desc, x["k_ctx"], x["v_ctx"], w.ctx_len, 0, layer.k_cache, layer.v_cache, w.ctx_len,
                           0)
        c.record()
        ts.append((a, c))
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(c) for a, c in ts[1:]]))


def query_step_timing(layer, x, w, reps: int, flush) -> dict:
    """The query step (append of the T0 query tokens, partials, merge) with L2
    and MALL evicted before each: through the three calls and through
    sa_phase2_step (one call). Medians in microseconds."""
    import torch
    from long_context_attention_amd import _binding as B
    t = w.n_query
    n = layer.n_parts * t * layer.hq
    op = layer._out_part[: n * layer.d].view(layer.n_parts, t, layer.hq, layer.d)
    lp = layer._lse_part[:n].view(layer.n_parts, t, layer.hq)
    q, k, v = x["q_qry"], x["k_qry"], x["v_qry"]
    res = {}
    for mode in ("calls", "fused", "calls", "fused"):
        ts = []
        for _ in range(reps):
            flush.sum()
            a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if mode == "calls":
                B.sa_decode_append(layer.desc, k, v, t, w.ctx_len, layer.k_tail, layer.v_tail, layer.tail_cap, 0)
                B.sa_phase2_partial(layer.desc, q, t, w.ctx_len, layer.k_cache, layer.v_cache, w.ctx_len,
                                    w.block_len, layer.k_tail, layer.v_tail, layer.tail_cap, t, w.ctx_len, op, lp,
                                    layer.workspace)
                B.sa_phase2_merge(layer.n_parts, t, layer.hq, layer.d, op, lp, layer.out[:t], layer.dtype,
                                  layer.lse[:t])
            else:
                B.sa_phase2_step(layer.desc, q, k, v, t, layer.k_cache, layer.v_cache, w.ctx_len, w.block_len,
                                 layer.k_tail, layer.v_tail, layer.tail_cap, 0, layer.out[:t], layer.lse[:t],
                                 layer.workspace)
            c.record()
            ts.append((a, c))
        torch.cuda.synchronize()
        res.setdefault(mode, []).extend(a.elapsed_time(c) * 1e3 for a, c in ts)
    return {"us_three_calls": round(float(np.median(res["calls"])), 2),
            "us_fused_call": round(float(np.median(res["fused"])), 2)}


def decode_step_fused_vs_calls(layer, x, w, reps: int, flush) -> dict:
    """A whole decode step (append + partial + merge) with the caches evicted
    before each: through the three calls, and through sa_phase2_step (one call,
    the chunk and partition merges in one launch). Medians in microseconds."""
    import torch
    from long_context_attention_amd import _binding as B
    t, tl = 1, w.n_query
    n = layer.n_parts * t * layer.hq
    op = layer._out_part[: n * layer.d].view(layer.n_parts, t, layer.hq, layer.d)
    lp = layer._lse_part[:n].view(layer.n_parts, t, layer.hq)
    q, k, v = x["q_dec"][:1], x["k_dec"][:1], x["v_dec"][:1]
    pos = w.ctx_len + tl
    res = {}
    for mode in ("calls", "fused", "calls", "fused"):
        ts = []
        for _ in range(reps):
            flush.sum()
            a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if mode == "calls":
                B.sa_decode_append(layer.desc, k, v, t, pos, layer.k_tail, layer.v_tail, layer.tail_cap, tl)
                B.sa_phase2_partial(layer.desc, q, t, pos, layer.k_cache, layer.v_cache, w.ctx_len, w.block_len,
                                    layer.k_tail, layer.v_tail, layer.tail_cap, tl + t, w.ctx_len, op, lp,
                                    layer.workspace)
                B.sa_phase2_merge(layer.n_parts, t, layer.hq, layer.d, op, lp, layer.out[:t], layer.dtype,
                                  layer.lse[:t])
            else:
                B.sa_phase2_step(layer.desc, q, k, v, t, layer.k_cache, layer.v_cache, w.ctx_len, w.block_len,
                                 layer.k_tail, layer.v_tail, layer.tail_cap, tl, layer.out[:t], layer.lse[:t],
                                 layer.workspace)
            c.record()
            ts.append((a, c))
        torch.cuda.synchronize()
        res.setdefault(mode, []).extend(a.elapsed_time(c) * 1e3 for a, c in ts)
    # Consecutive steps between one pair of events, alternating between this
    # layer's caches and a copy (each 537 MB at 128K, more than L2 + MALL, so
    # every step streams from HBM as a model's successive layers would): the
    # cost of the timing events themselves is spread over the steps.
    kc2, vc2 = layer.k_cache.clone(), layer.v_cache.clone()
    caches = [(layer.k_cache, layer.v_cache), (kc2, vc2)]
    n_b2b = 16
    b2b, b2b_pm = [], []
    for _ in range(3):
        flush.sum()
        a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n_b2b):
            kc, vc = caches[i % 2]
            B.sa_phase2_step(layer.desc, q, k, v, t, kc, vc, w.ctx_len, w.block_len, layer.k_tail, layer.v_tail,
                             layer.tail_cap, tl, layer.out[:t], layer.lse[:t], layer.workspace)
        c.record()
        torch.cuda.synchronize()
        b2b.append(a.elapsed_time(c) * 1e3 / n_b2b)
        # the headline's partial + merge (the tail already holds the step's row), the same way
        flush.sum()
        a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(n_b2b):
            kc, vc = caches[i % 2]
            B.sa_phase2_partial(layer.desc, q, t, pos, kc, vc, w.ctx_len, w.block_len, layer.k_tail, layer.v_tail,
                                layer.tail_cap, tl + t, w.ctx_len, op, lp, layer.workspace)
            B.sa_phase2_merge(layer.n_parts, t, layer.hq, layer.d, op, lp, layer.out[:t], layer.dtype, layer.lse[:t])
        c.record()
        torch.cuda.synchronize()
        b2b_pm.append(a.elapsed_time(c) * 1e3 / n_b2b)
    del kc2, vc2, caches
    # Two events with nothing between them: what one timed interval adds.
    ev = []
    for _ in range(reps):
        a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        c.record()
        ev.append((a, c))
    torch.cuda.synchronize()
    return {"decode_step_us_three_calls": round(float(np.median(res["calls"])), 2),
            "decode_step_us_fused_call": round(float(np.median(res["fused"])), 2),
            "decode_step_us_fused_back_to_back": round(float(np.median(b2b)), 2),
            "decode_us_partial_merge_back_to_back": round(float(np.median(b2b_pm)), 2),
            "empty_event_pair_us": round(float(np.median([a.elapsed_time(c) * 1e3 for a, c in ev])), 2),
            "note": "append + partial + merge with L2/MALL evicted before each step; fused = sa_phase2_step; "
                    "back_to_back = 16 consecutive sa_phase2_step calls (or partial + merge calls) between one pair "
                    "of events, alternating between two copies of the caches (each larger than L2 + MALL), per step"}


def batched_decode(n_seq: int, flush, reps: int = 10) -> dict:
    """Decode steps of n_seq Llama-8B-shaped sequences at 32K context (each its own
    cache and tail, after its query step), caches evicted before each timed step:
    n_seq sa_phase2_step calls against one sa_decode_step_batched call."""
    import torch
    from long_context_attention_amd import _binding as B
    from long_context_attention_amd.runner import StarLayer
    w = W.LLAMA8B_32K
    x = {k: to_device(v) for k, v in W.all_tensors(w, 0).items()}
    layers = []
    for _ in range(n_seq):
        l_ = StarLayer.for_workload(w)
        l_.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
        l_.step(x["q_qry"], x["k_qry"], x["v_qry"])
        layers.append(l_)
    tl = w.n_query
    q, k, v = x["q_dec"][0], x["k_dec"][0], x["v_dec"][0]
    seqs = [dict(q=q, k_new=k, v_new=v, k_cache=l_.k_cache, v_cache=l_.v_cache, k_tail=l_.k_tail, v_tail=l_.v_tail,
                 out=l_.out[0], lse=l_.lse[0], ctx_len=w.ctx_len, block_len=w.block_len, tail_cap=l_.tail_cap,
                 tail_len=tl) for l_ in layers]
    arr = B.decode_seqs(seqs)
    ws = torch.empty(B.sa_decode_batch_workspace_bytes(layers[0].desc, arr), dtype=torch.uint8, device="cuda")
    res = {}
    for mode in ("one", "single", "batched", "one", "single", "batched"):
        ts = []
        for _ in range(reps):
            flush.sum()
            a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if mode == "one":
                l_ = layers[0]
                B.sa_phase2_step(l_.desc, q[None], k[None], v[None], 1, l_.k_cache, l_.v_cache, w.ctx_len,
                                 w.block_len, l_.k_tail, l_.v_tail, l_.tail_cap, tl, l_.out[:1], l_.lse[:1],
                                 l_.workspace)
            elif mode == "single":
                for l_ in layers:
                    B.sa_phase2_step(l_.desc, q[None], k[None], v[None], 1, l_.k_cache, l_.v_cache, w.ctx_len,
                                     w.block_len, l_.k_tail, l_.v_tail, l_.tail_cap, tl, l_.out[:1], l_.lse[:1],
                                     l_.workspace)
            else:
                B.sa_decode_step_batched(layers[0].desc, arr, ws)
            c.record()
            ts.append((a, c))
        torch.cuda.synchronize()
        res.setdefault(mode, []).extend(a.elapsed_time(c) * 1e3 for a, c in ts)
    step_bytes = n_seq * acc.phase2_step_bytes(w.ctx_len, w.n_query + 1, 1, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                               w.elem_bytes)
    us_s, us_b = float(np.median(res["single"])), float(np.median(res["batched"]))
    us_1 = float(np.median(res["one"]))
    one_bytes = acc.phase2_step_bytes(w.ctx_len, w.n_query + 1, 1, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                      w.elem_bytes)
    del layers, x, ws
    torch.cuda.empty_cache()
    return {"workload": f"{n_seq} x {w.name}", "n_seq": n_seq, "step_bytes": int(step_bytes),
            "us_per_step_separate_calls": round(us_s, 2), "us_per_step_batched": round(us_b, 2),
            "gbps_separate_calls": round(step_bytes / (us_s * 1e-6) / 1e9, 1),
            "gbps_batched": round(step_bytes / (us_b * 1e-6) / 1e9, 1),
            "one_sequence_fused_step_us": round(us_1, 2),
            "one_sequence_fused_step_gbps": round(one_bytes / (us_1 * 1e-6) / 1e9, 1),
            "note": "one decode step (append + partials + merge) of every sequence, caches evicted before each"}


def machine_ceilings() -> dict:
    """Measured streaming-read bandwidth and dense bf16 MFMA rate of this GPU."""
    import torch
    from long_context_attention_amd import _binding as B
    buf = torch.ones(1 << 29, dtype=torch.int32, device="cuda")          # 2 GiB
    sink = torch.zeros(256, dtype=torch.float32, device="cuda")
    B.sa_calibrate_stream_read(buf, sink)
    ts = []
    for _ in range(5):
        a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        B.sa_calibrate_stream_read(buf, sink)
        c.record()
        ts.append((a, c))
    torch.cuda.synchronize()
    read_ms = float(np.median([a.elapsed_time(c) for a, c in ts]))
    iters, wgs = 2000, 256 * 4
    B.sa_calibrate_mfma(iters, wgs, sink)
    a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    B.sa_calibrate_mfma(iters, wgs, sink)
    c.record()
    torch.cuda.synchronize()
    mfma_ms = a.elapsed_time(c)
    del buf
    info = B.sa_device_info()
    return {"hbm_read_gbps": round((1 << 31) / (read_ms * 1e-3) / 1e9, 1),
            "mfma_bf16_tflops": round(wgs * 4 * iters * 8 * 32768 / (mfma_ms * 1e-3) / 1e12, 1),
            # the vendor peaks re-derived from the device's own properties: CUs x peak clock x 4096 dense bf16
            # FLOP per clock per CU, and HBM3E's 4 transfers per pin per reported memory clock over the bus width
            "device": {**info,
                       "bf16_tflops_from_clock": round(info["n_cus"] * info["clock_khz"] * 1e3 * 4096 / 1e12, 1),
                       "hbm_gbps_from_clock": round(4 * info["mem_clock_khz"] * 1e3 * info["mem_bus_bits"] / 8 / 1e9,
                                                    1)}}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_llama8b_128k.md")


def sources_sha256(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def profiled_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary, or None if there is none or its kernel sources changed."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    m = re.search(r"```json\n(.*?)\n```", open(TRAFFIC_FILE).read(), re.S)
    if not m:
        return None
    for rec in json.loads(m.group(1)):
        if rec["kernel"] == kernel and rec["workload"] == workload:
            if sources_sha256(rec["sources"]) != rec["sources_sha256"]:
                return None
            return int(rec["bytes_per_launch"])
    return None


def star_vs_global(layer, x, w, star_ms: float) -> dict:
    """Exact causal attention over the whole context (the Phase-1 kernel with a
    single block) against Star Attention's context outputs."""
    import torch
    from long_context_attention_amd.runner import StarLayer
    gw = w.with_block(w.ctx_len)
    gl = StarLayer.for_workload(gw, max_t_q=1)
    gl.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
    a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    gl.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
    c.record()
    torch.cuda.synchronize()
    g_ms = a.elapsed_time(c)
    b = w.block_len
    dev_max, dev_sum, n_el = 0.0, 0.0, 0
    for i in range(2, w.n_blocks):     # blocks 1 and 2 (0-based 0, 1) are exact by construction
        d = (layer.out_ctx[i * b:(i + 1) * b].float() - gl.out_ctx[i * b:(i + 1) * b].float()).abs()
        dev_max = max(dev_max, float(d.max()))
        dev_sum += float(d.sum())
        n_el += d.numel()
        del d
    exact01 = float((layer.out_ctx[:2 * b].float() - gl.out_ctx[:2 * b].float()).abs().max()) \
        if w.n_blocks >= 2 else float((layer.out_ctx.float() - gl.out_ctx.float()).abs().max())
    g_flops = acc.global_causal_flops(w.ctx_len, w.n_q_heads, w.head_dim)
    p_flops = acc.phase1_flops(w.ctx_len, w.block_len, w.anchor_len, w.n_q_heads, w.head_dim)

    def anchor_variant(vw, anchor_pos=None) -> dict:
        """One of the paper's anchor ablations (same useful work), timed like Phase 1,
        with its deviation from exact global attention in blocks >= 3."""
        vl = StarLayer.for_workload(vw, max_t_q=1, anchor_pos=anchor_pos)
        vl.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
        a.record()
        vl.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
        c.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(c)
        v_max, v_sum = 0.0, 0.0
        for i in range(2, w.n_blocks):
            d = (vl.out_ctx[i * b:(i + 1) * b].float() - gl.out_ctx[i * b:(i + 1) * b].float()).abs()
            v_max = max(v_max, float(d.max()))
            v_sum += float(d.sum())
            del d
        del vl
        return {"phase1_ms": round(ms, 3), "phase1_tflops": round(p_flops / (ms * 1e-3) / 1e12, 2),
                "max_abs_dev_blocks_ge3": v_max, "mean_abs_dev_blocks_ge3": v_sum / max(n_el, 1)}

    # the previous block as anchor; the first block's anchor at random position IDs
    # from the prefix (seeded; the rotated anchor keys are written inside the timed call)
    prev = anchor_variant(w.with_anchor("previous"))
    rw = w.with_anchor_at("random")
    rand = anchor_variant(rw, W.anchor_positions(rw))
    del gl
    torch.cuda.empty_cache()
    return {"global_ms": round(g_ms, 3), "global_tflops": round(g_flops / (g_ms * 1e-3) / 1e12, 2),
            "phase1_speedup_vs_global": round(g_ms / star_ms, 3),
            "max_abs_dev_blocks_ge3": dev_max, "mean_abs_dev_blocks_ge3": dev_sum / max(n_el, 1),
            "max_abs_diff_blocks_1_2": exact01,
            "previous_block_anchor": prev, "random_prefix_anchor_positions": rand,
            "note": "context only: Star Attention approximates global attention for blocks >= 3"}


def _blas_threads() -> tuple[int, int]:
    """(threads the oracle's BLAS uses, host cores visible to this process). The
    threads are the visible cores, capped by OMP_NUM_THREADS where the job sets
    one (a GPU machine gives each GPU a share of its host cores)."""
    visible = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return (min(visible, int(cap)) if cap.isdigit() and int(cap) > 0 else visible), visible


def _oracle_phase1_rows(w: W.Workload, x: dict, rows: np.ndarray, blocks: list) -> tuple[int, float]:
    """The oracle's Phase 1 for the given rows of the given blocks, every query
    head (one KV head at a time); returns (useful FLOP of those rows, seconds)."""
    import oracle as O
    b, A, g = w.block_len, w.anchor_len, w.group
    flops, dt = 0, 0.0
    for kvh in range(w.n_kv_heads):
        hs, ks = slice(kvh * g, (kvh + 1) * g), slice(kvh, kvh + 1)
        for i in blocks:
            tok, n_anc = O.augmented_block(i, b, A)
            sel = n_anc + rows
            n_keys = int(sel.max()) + 1
            qf = W.to_f64(x["q_ctx"][tok[sel]][:, hs])
            kf = W.to_f64(x["k_ctx"][tok[:n_keys]][:, ks])
            vf = W.to_f64(x["v_ctx"][tok[:n_keys]][:, ks])
            t0 = time.perf_counter()
            O.phase1_block(_Rows(qf, tok[sel]), _Rows(kf, tok[:n_keys]), _Rows(vf, tok[:n_keys]), i, b, A,
                           w.rope_theta, w.softmax_scale, rows=rows)
            dt += time.perf_counter() - t0
            flops += 4 * w.head_dim * g * int((sel + 1).sum())
    return flops, dt


def _oracle_phase2_step(w: W.Workload, x: dict, t: int) -> float:
    """Seconds of one whole Phase-2 step of the oracle (every partition's partial
    and the merge, all KV heads) for t new tokens: the query step (t = T0) or the
    first decode step (t = 1, after the query step). The context cache is
    prepared (RoPE'd) outside the timed region, as Phase 1 would leave it."""
    import oracle as O
    g = w.group
    if t == w.n_query:
        q, kq, vq, q_pos = x["q_qry"], x["k_qry"], x["v_qry"], w.ctx_len
    else:
        q = x["q_dec"][:1]
        kq = np.concatenate([x["k_qry"], x["k_dec"][:1]])
        vq = np.concatenate([x["v_qry"], x["v_dec"][:1]])
        q_pos = w.ctx_len + w.n_query
    pos = np.arange(w.ctx_len)
    dt = 0.0
    for kvh in range(w.n_kv_heads):
        hs, ks = slice(kvh * g, (kvh + 1) * g), slice(kvh, kvh + 1)
        kc = O.rope(W.to_f64(x["k_ctx"][:, ks]), pos, w.rope_theta)
        vc = W.to_f64(x["v_ctx"][:, ks])
        t1 = time.perf_counter()
        kt, vt = O.tail_keys(W.to_f64(kq[:, ks]), W.to_f64(vq[:, ks]), w.ctx_len, w.rope_theta)
        op, lp = O.phase2_partials(W.to_f64(q[:, hs]), q_pos, kc, vc, w.block_len, kt, vt, w.ctx_len,
                                   w.rope_theta, w.softmax_scale)
        O.merge(op, lp)
        dt += time.perf_counter() - t1
        del kc, vc
    return dt


def _oracle_full_layer(w: W.Workload) -> dict:
    """The oracle on a whole small layer: Phase 1 over every context row, the
    query step and every decode step (seconds of each)."""
    import oracle as O
    x = W.all_tensors(w, 0)
    f = {k: W.to_f64(v) for k, v in x.items()}
    t0 = time.perf_counter()
    p1 = O.phase1(f["q_ctx"], f["k_ctx"], f["v_ctx"], w.block_len, w.anchor_len, w.rope_theta, w.softmax_scale)
    t1 = time.perf_counter()
    kt, vt = O.tail_keys(np.concatenate([f["k_qry"], f["k_dec"]]), np.concatenate([f["v_qry"], f["v_dec"]]),
                         w.ctx_len, w.rope_theta)
    T0 = w.n_query
    op, lp = O.phase2_partials(f["q_qry"], w.ctx_len, p1["k_cache"], p1["v_cache"], w.block_len, kt[:T0], vt[:T0],
                               w.ctx_len, w.rope_theta, w.softmax_scale)
    O.merge(op, lp)
    t2 = time.perf_counter()
    for s in range(w.n_decode):
        n = T0 + s + 1
        op, lp = O.phase2_partials(f["q_dec"][s:s + 1], w.ctx_len + T0 + s, p1["k_cache"], p1["v_cache"],
                                   w.block_len, kt[:n], vt[:n], w.ctx_len, w.rope_theta, w.softmax_scale)
        O.merge(op, lp)
    t3 = time.perf_counter()
    flops = acc.phase1_flops(w.ctx_len, w.block_len, w.anchor_len, w.n_q_heads, w.head_dim)
    return {"workload": w.name, "phase1_s": round(t1 - t0, 3), "phase1_tflops": round(flops / (t1 - t0) / 1e12, 5),
            "query_step_s": round(t2 - t1, 4), "decode_steps_s": round(t3 - t2, 4), "decode_steps": w.n_decode,
            "note": "the oracle's own Phase 1 computes the anchor rows of every augmented block too (it follows "
                    "the pages' definition literally); the FLOP rate counts the useful work only"}


def cpu_baseline(w: W.Workload) -> dict:
    """The fp64 oracle, as it stands, on bounded samples of the same workload: a
    Phase-1 row sample on every thread and on one thread, one query step, one
    decode step, and the small float32 workload in full."""
    from threadpoolctl import threadpool_limits
    threads, visible = _blas_threads()
    x = {k: W.tensor(w, t, 0) for k, t in (("q_ctx", W.T_Q_CTX), ("k_ctx", W.T_K_CTX), ("v_ctx", W.T_V_CTX),
                                           ("q_qry", W.T_Q_QRY), ("k_qry", W.T_K_QRY), ("v_qry", W.T_V_QRY),
                                           ("q_dec", W.T_Q_DEC), ("k_dec", W.T_K_DEC), ("v_dec", W.T_V_DEC))}
    b = w.block_len
    blocks = [2, w.n_blocks] if w.n_blocks > 1 else [1]

    def rows_of(n_spread):
        return np.unique(np.concatenate([[0, 1, b - 2, b - 1], np.linspace(0, b - 1, n_spread).astype(np.int64)]))

    rows, rows1 = rows_of(560), rows_of(36)
    with threadpool_limits(limits=threads):
        flops, dt = _oracle_phase1_rows(w, x, rows, blocks)
        dec_s = _oracle_phase2_step(w, x, 1)
        qry_s = _oracle_phase2_step(w, x, w.n_query)
        small = _oracle_full_layer(W.SMALL_F32)
    with threadpool_limits(limits=1):
        flops1, dt1 = _oracle_phase1_rows(w, x, rows1, blocks)
    dec_bytes = acc.phase2_step_bytes(w.ctx_len, w.n_query + 1, 1, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                      w.elem_bytes)
    q_bytes = acc.phase2_step_bytes(w.ctx_len, w.n_query, w.n_query, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                    w.elem_bytes)
    q_flops = acc.phase2_step_flops(w.ctx_len, w.n_query, w.n_query, w.n_q_heads, w.head_dim)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "cores_visible": int(visible),
            "kind": "oracle",
            "sample": f"Phase-1 oracle (numpy fp64) for {len(rows)} rows of blocks {blocks} (560 evenly spaced over "
                      f"[0, b) plus the first and last two), all {w.n_q_heads} query heads; {flops / 1e9:.2f} GFLOP "
                      f"useful in {dt:.1f} s on {threads} threads",
            "seconds": dt,
            "one_thread": {"value": flops1 / dt1 / 1e12, "unit": "TFLOP/s", "cores": 1, "seconds": round(dt1, 3),
                           "sample": f"the same for {len(rows1)} rows (36 evenly spaced plus the first and last two) "
                                     f"of blocks {blocks}; {flops1 / 1e9:.2f} GFLOP"},
            "phase2_decode_step": {"seconds": round(dec_s, 3), "gbps_equivalent": round(dec_bytes / dec_s / 1e9, 3),
                                   "sample": "one whole decode step (every partition's partial and the merge), "
                                             "all KV heads, cache prepared outside the timed region"},
            "query_step": {"seconds": round(qry_s, 3), "gbps_equivalent": round(q_bytes / qry_s / 1e9, 3),
                           "tflops": round(q_flops / qry_s / 1e12, 5),
                           "sample": f"one whole query step ({w.n_query} tokens: every partition's partial and the "
                                     "merge), all KV heads, cache prepared outside the timed region"},
            "small_f32_2k_full": small}


class _Rows:
    """Maps token indices of one augmented block onto pre-gathered rows."""

    def __init__(self, data, toks):
        self.data = data
        self.pos = {int(t): j for j, t in enumerate(toks)}
        self.shape = (max(self.pos) + 1,) + data.shape[1:]

    def __getitem__(self, idx):
        return self.data[[self.pos[int(t)] for t in np.atleast_1d(idx)]]


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="llama8b_128k", choices=sorted(W.WORKLOADS))
    ap.add_argument("--block", type=int, default=None, help="block length b (default: the workload's)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the block-size sweep of the 128K workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-global", action="store_true", help="skip the Star-vs-exact-global comparison")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-batch", action="store_true", help="skip the batched multi-sequence decode leg")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the Star Attention hot path here runs its block partitions on a "
              "single MI355X. Across GPUs the blocks would shard with no communication in Phase 1 and one "
              "(output, LSE) exchange per token in Phase 2; that path is not built.", file=sys.stderr)
        return 2

    import torch
    from long_context_attention_amd.runner import StarLayer
    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    w = W.WORKLOADS[args.workload]
    if args.block:
        w = w.with_block(args.block)
    log(f"workload {w.name}: L={w.ctx_len} b={w.block_len} A={w.anchor_len} Hq={w.n_q_heads} Hkv={w.n_kv_heads} "
        f"d={w.head_dim} T0={w.n_query} S={w.n_decode}")
    t0 = time.time()
    xh = W.all_tensors(w, args.seed)
    x = {k: to_device(v) for k, v in xh.items()}
    log(f"inputs generated and resident in HBM ({time.time() - t0:.1f}s)")
    layer = StarLayer.for_workload(w)

    run_steps(layer, x, w, args.warmup, record=False)
    log("warmup done")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    rec = run_steps(layer, x, w, args.steps, record=True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    log(f"timed {args.steps} steps in {wall:.3f}s")

    p1_flops = acc.phase1_flops(w.ctx_len, w.block_len, w.anchor_len, w.n_q_heads, w.head_dim)
    p1_ms = float(np.mean([r["p1"] for r in rec]))
    p1_tflops = p1_flops / (p1_ms * 1e-3) / 1e12
    dec_ms = [d for r in rec for d in r["d"]]
    dec_bytes = float(np.mean([acc.phase2_step_bytes(w.ctx_len, w.n_query + s + 1, 1, w.n_q_heads, w.n_kv_heads,
                                                     w.head_dim, w.elem_bytes) for s in range(w.n_decode)]))
    dec_step_ms = float(np.mean(dec_ms))
    q_ms = float(np.mean([r["q"] for r in rec]))
    q_bytes = acc.phase2_step_bytes(w.ctx_len, w.n_query, w.n_query, w.n_q_heads, w.n_kv_heads, w.head_dim,
                                    w.elem_bytes)
    q_flops = acc.phase2_step_flops(w.ctx_len, w.n_query, w.n_query, w.n_q_heads, w.head_dim)

    # Phase-2 decode partial + merge alone (tail already appended), without and with an L2/MALL flush.
    p2 = phase2_only(layer, x, w, 20)
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")   # 1 GiB > L2 + MALL
    p2f = phase2_only(layer, x, w, 10, flush)
    p2w_ms = float(np.median(p2))          # caches warm from the previous step
    p2_ms = float(np.median(p2f))          # caches evicted: the headline
    p2_gbps = dec_bytes / (p2_ms * 1e-3) / 1e9
    log(f"phase 1: {p1_ms:.2f} ms, {p1_tflops:.1f} TFLOP/s; decode partial+merge {p2_ms * 1e3:.1f} us "
        f"({p2_gbps:.0f} GB/s), warm {p2w_ms * 1e3:.1f} us; query step {q_ms:.2f} ms")
    fused = decode_step_fused_vs_calls(layer, x, w, 10, flush) if w.dtype == "bf16" else None
    if fused:
        log(f"decode step incl. append, caches evicted: three calls {fused['decode_step_us_three_calls']} us, "
            f"sa_phase2_step {fused['decode_step_us_fused_call']} us, back to back "
            f"{fused['decode_step_us_fused_back_to_back']} us per step (partial + merge "
            f"{fused['decode_us_partial_merge_back_to_back']} us); empty event pair {fused['empty_event_pair_us']} us")
    qstep = query_step_timing(layer, x, w, 6, flush)
    q_us = min(qstep["us_three_calls"], qstep["us_fused_call"])
    log(f"query step, caches evicted: three calls {qstep['us_three_calls']} us, sa_phase2_step "
        f"{qstep['us_fused_call']} us")
    rope_ms = rope_cache_ms(layer, x, w)
    attn_ms = p1_ms - rope_ms
    attn_tflops = p1_flops / (attn_ms * 1e-3) / 1e12
    log(f"phase 1 RoPE/cache kernel {rope_ms:.3f} ms; attention kernel {attn_ms:.2f} ms ({attn_tflops:.1f} TFLOP/s)")

    sweep = []
    if not args.no_sweep and w.name.startswith("llama8b_128k"):
        for bw in W.LLAMA8B_128K_SWEEP:
            if bw.block_len == w.block_len:
                sweep.append({"block_len": bw.block_len, "n_blocks": bw.n_blocks, "phase1_ms": p1_ms,
                              "phase1_tflops": p1_tflops, "decode_us": p2_ms * 1e3, "decode_gbps": p2_gbps})
                continue
            ls = StarLayer.for_workload(bw)
            ls.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
            ls.step(x["q_qry"], x["k_qry"], x["v_qry"])
            torch.cuda.synchronize()
            ts = []
            for _ in range(2):
                a, c = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                ls.encode(x["q_ctx"], x["k_ctx"], x["v_ctx"])
                c.record()
                ts.append((a, c))
            ls.step(x["q_qry"], x["k_qry"], x["v_qry"])
            d_ms = float(np.median(phase2_only(ls, x, bw, 10, flush)))
            ms = float(np.median([a.elapsed_time(c) for a, c in ts]))
            fl = acc.phase1_flops(bw.ctx_len, bw.block_len, bw.anchor_len, bw.n_q_heads, bw.head_dim)
            sweep.append({"block_len": bw.block_len, "n_blocks": bw.n_blocks, "phase1_ms": ms,
                          "phase1_tflops": fl / (ms * 1e-3) / 1e12, "decode_us": d_ms * 1e3,
                          "decode_gbps": dec_bytes / (d_ms * 1e-3) / 1e9})
            log(f"sweep b={bw.block_len}: phase 1 {ms:.2f} ms ({sweep[-1]['phase1_tflops']:.1f} TFLOP/s), "
                f"decode {d_ms * 1e3:.1f} us")
            del ls
        sweep.sort(key=lambda s: s["block_len"])
    del flush

    result = {
        "metric": METRIC,
        "value": round(p1_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic: seeded i.i.d. N(0,1) Q/K/V (bf16), keys of positions 0-3 shifted +3 along a seeded "
                "unit direction; no trained weights",
        "config": {"workload": w.name, "ctx_len": w.ctx_len, "block_len": w.block_len, "anchor_len": w.anchor_len,
                   "n_blocks": w.n_blocks, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
                   "head_dim": w.head_dim, "query_tokens": w.n_query, "decode_steps": w.n_decode,
                   "rope_theta": w.rope_theta},
        "phase1": {"ms": round(p1_ms, 3), "useful_flop": p1_flops, "tflops": round(p1_tflops, 2),
                   "frac_of_bf16_peak": round(p1_tflops / PEAK_BF16_TFLOPS, 4),
                   "rope_cache_kernel_ms": round(rope_ms, 3), "attention_kernel_ms": round(attn_ms, 3),
                   "attention_kernel_tflops": round(attn_tflops, 2),
                   "note": "ms = the whole sa_phase1_encode call (RoPE/cache kernel, job-counter reset, attention "
                           "kernel); attention_kernel_ms = ms minus the RoPE/cache kernel timed alone with the same "
                           "arguments"},
        "phase2": {"value": round(p2_gbps, 1), "unit": "GB/s", "decode_us": round(p2_ms * 1e3, 2),
                   "decode_us_warm_caches": round(p2w_ms * 1e3, 2),
                   "decode_gbps_warm_caches": round(dec_bytes / (p2w_ms * 1e-3) / 1e9, 1),
                   "decode_step_us_incl_append": round(dec_step_ms * 1e3, 2),
                   "decode_bytes": int(dec_bytes), "frac_of_hbm_peak": round(p2_gbps / PEAK_HBM_GBPS, 4),
                   "query_step_ms": round(q_ms, 3), "query_step_bytes": int(q_bytes), "query_step_flop": q_flops,
                   "query_step_cold": qstep},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": profiled_traffic("attn_tile_kernel<128, 0>", w.name),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE)",
                     "kernel": "attn_tile_kernel<128, 0>: useful FLOP per launch / the attention kernel's time "
                               "(phase1.attention_kernel_ms); value counts the whole call"},
        "roofline_query": {"bound": "hbm", "achieved": round(q_bytes / (q_us * 1e-6) / 1e9, 1), "peak": PEAK_HBM_GBPS,
                           "unit": "GB/s", "frac": round(q_bytes / (q_us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                           "achieved_tflops": round(q_flops / (q_us * 1e-6) / 1e12, 1),
                           "frac_of_bf16_peak": round(q_flops / (q_us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
                           "us": q_us, "traffic": profiled_traffic("attn_tile_kernel<128, 1>", w.name),
                           "traffic_unit": "HBM bytes per launch of the query-step tile kernel",
                           "kernel": "the whole query step (append, attn_tile_kernel<128, 1>, merge) with caches "
                                     "evicted, the faster of the three calls and sa_phase2_step; arithmetic "
                                     "intensity below the ridge point, so HBM is the nominal bound"},
        "roofline_phase2": {"bound": "hbm", "achieved": round(p2_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                            "frac": round(p2_gbps / PEAK_HBM_GBPS, 4),
                            "traffic": profiled_traffic("phase2_decode_kernel<128, 4, 32>", w.name),
                            "traffic_unit": "HBM bytes per launch of the decode kernel",
                            "kernel": "decode step: sa_phase2_partial (phase2_decode_kernel + chunk merge) "
                                      "+ sa_phase2_merge, caches evicted",
                            "fused_step_achieved": (round(dec_bytes / (fused["decode_step_us_fused_call"] * 1e-6) / 1e9,
                                                          1) if fused else None),
                            "fused_step_frac": (round(dec_bytes / (fused["decode_step_us_fused_call"] * 1e-6) / 1e9
                                                      / PEAK_HBM_GBPS, 4) if fused else None),
                            "back_to_back_frac": (round(
                                dec_bytes / (fused["decode_us_partial_merge_back_to_back"] * 1e-6) / 1e9
                                / PEAK_HBM_GBPS, 4) if fused else None),
                            "fused_step_back_to_back_frac": (round(
                                dec_bytes / (fused["decode_step_us_fused_back_to_back"] * 1e-6) / 1e9
                                / PEAK_HBM_GBPS, 4) if fused else None),
                            "fused_step_note": "fused_step: the same step through sa_phase2_step, the append "
                                               "included; back_to_back: consecutive steps over two cache copies, "
                                               "per step, without one timing event's idle gap"},
        "sweep": sweep,
    }
    if fused:
        result["phase2"]["fused_step"] = fused
    if not args.no_batch and w.dtype == "bf16":
        log("batched decode of 8 sequences at 32K ...")
        flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        result["phase2"]["batched_decode"] = batched_decode(8, flush)
        del flush
        log(f"batched decode: {result['phase2']['batched_decode']}")
    if not args.no_global:
        log("star vs exact global attention ...")
        result["star_vs_global"] = star_vs_global(layer, x, w, p1_ms)
        log(f"star vs global: {result['star_vs_global']}")
    result["measured_ceilings"] = machine_ceilings()
    log(f"measured ceilings: {result['measured_ceilings']}")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(w)
        cb = result["cpu_baseline"]
        log(f"cpu baseline: {cb['value']:.4f} TFLOP/s on {cb['cores']} threads ({cb['seconds']:.1f}s); one thread "
            f"{cb['one_thread']['value']:.5f} TFLOP/s; query step {cb['query_step']['seconds']} s; decode step "
            f"{cb['phase2_decode_step']['seconds']} s; {cb['small_f32_2k_full']}")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
