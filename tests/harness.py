"""Shared test plumbing: run one workload through libstarattn and through the oracle.

The GPU side goes through the C ABI (via ``long_context_attention_amd.runner``);
the oracle side uses only ``oracle`` and the seeded inputs of ``workloads``.
Large workloads are checked on a seeded sample of context rows (every block's
rows 0, 1, b/2, b-2, b-1 plus random rows) and on every Phase-2 row; the oracle
runs one KV head (and its query heads) at a time to bound host memory.
"""
from __future__ import annotations

import dataclasses
import os
import sys
import time

import numpy as np

import oracle as O
import workloads as W

# Tolerances of the Star Attention hot path (max abs for float32 workloads; max
# and mean abs for bf16 workloads).
TOL = {"f32": {"max": 1e-4, "mean": None}, "bf16": {"max": 2e-2, "mean": 2e-3}}


def log(msg: str) -> None:
    print(f"[harness {time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


class F64View:
    """Row-indexable float64 view of a workload tensor slice (converts on access)."""

    def __init__(self, arr: np.ndarray, heads: slice):
        self.a, self.heads = arr, heads
        self.shape = (arr.shape[0], len(range(*heads.indices(arr.shape[1]))), arr.shape[2])

    def __getitem__(self, idx):
        return W.to_f64(self.a[idx][:, self.heads])


def to_device(arr: np.ndarray, device="cuda"):
    import torch
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(arr).to(device)


def to_host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


@dataclasses.dataclass
class GpuResult:
    out_ctx: dict            # block -> [rows, Hq, d]
    k_cache: np.ndarray      # [Hkv, n_rows_sampled, d] for sampled rows (positions in cache_rows)
    v_cache: np.ndarray
    cache_rows: np.ndarray
    qry: dict                # out, lse, out_part, lse_part
    dec: list                # per decode step: dict as qry
    k_tail: np.ndarray = None   # [Hkv, T0 + S, d]: the tail rows the steps appended
    v_tail: np.ndarray = None


def run_gpu(w: W.Workload, x: dict, rows_by_block: dict, cache_rows: np.ndarray, device="cuda") -> GpuResult:
    import torch
    from long_context_attention_amd.runner import StarLayer
    layer = StarLayer.for_workload(w, device=device, anchor_pos=W.anchor_positions(w))
    d = {k: to_device(v, device) for k, v in x.items()}
    # Every output starts as NaN: a row or tile the kernels never write shows up.
    for t in (layer.out_ctx, layer.k_cache, layer.v_cache, layer.k_tail, layer.v_tail):
        t.fill_(float("nan"))
    log(f"{w.name}: phase 1 (L={w.ctx_len}, b={w.block_len}, A={w.anchor_len}, anchor={w.anchor}, "
        f"anchor_at={w.anchor_at})")
    layer.encode(d["q_ctx"], d["k_ctx"], d["v_ctx"])
    torch.cuda.synchronize()
    for name in ("out_ctx", "k_cache", "v_cache"):
        assert bool(torch.isfinite(getattr(layer, name)).all()), f"{w.name}: {name} holds unwritten (NaN) elements"
    out_ctx = {}
    for i, rows in rows_by_block.items():
        idx = torch.as_tensor((i - 1) * w.block_len + rows, device=device)
        out_ctx[i] = to_host(layer.out_ctx.index_select(0, idx))
    ci = torch.as_tensor(cache_rows, device=device)
    kc = to_host(layer.k_cache.index_select(1, ci))
    vc = to_host(layer.v_cache.index_select(1, ci))
    log(f"{w.name}: query step (T0={w.n_query})")
    o, l_, op, lp = layer.step(d["q_qry"], d["k_qry"], d["v_qry"])
    qry = {"out": to_host(o), "lse": to_host(l_), "out_part": to_host(op), "lse_part": to_host(lp)}
    dec = []
    for s in range(w.n_decode):
        o, l_, op, lp = layer.step(d["q_dec"][s:s + 1], d["k_dec"][s:s + 1], d["v_dec"][s:s + 1])
        dec.append({"out": to_host(o), "lse": to_host(l_), "out_part": to_host(op), "lse_part": to_host(lp)})
    torch.cuda.synchronize()
    n_new = w.n_query + w.n_decode
    kt, vt = to_host(layer.k_tail[:, :n_new]), to_host(layer.v_tail[:, :n_new])
    log(f"{w.name}: gpu done")
    del layer, d
    torch.cuda.empty_cache()
    return GpuResult(out_ctx, kc, vc, cache_rows, qry, dec, kt, vt)


def run_oracle(w: W.Workload, x: dict, rows_by_block: dict, cache_rows: np.ndarray) -> dict:
    """Oracle outputs on the same inputs, one KV head group at a time."""
    g = w.group
    f = {k: v for k, v in x.items()}
    n = w.n_blocks
    out_ctx = {i: np.zeros((len(r), w.n_q_heads, w.head_dim)) for i, r in rows_by_block.items()}
    kc = np.zeros((w.n_kv_heads, len(cache_rows), w.head_dim))
    vc = np.zeros_like(kc)
    T0, S = w.n_query, w.n_decode
    n_rows = T0 + S
    opart = np.zeros((n + 1, n_rows, w.n_q_heads, w.head_dim))
    lpart = np.zeros((n + 1, n_rows, w.n_q_heads))
    k_tail = np.zeros((w.n_kv_heads, n_rows, w.head_dim))
    v_tail = np.zeros_like(k_tail)
    for kvh in range(w.n_kv_heads):
        hs = slice(kvh * g, (kvh + 1) * g)
        ks = slice(kvh, kvh + 1)
        q_ctx = F64View(f["q_ctx"], hs)
        k_ctx = F64View(f["k_ctx"], ks)
        v_ctx = F64View(f["v_ctx"], ks)
        p1 = O.phase1(q_ctx, k_ctx, v_ctx, w.block_len, w.anchor_len, w.rope_theta, w.softmax_scale,
                      rows_by_block=rows_by_block, anchor=w.anchor, anchor_pos=W.anchor_positions(w))
        for i in rows_by_block:
            out_ctx[i][:, hs] = p1["out"][i]
        kc[kvh] = p1["k_cache"][cache_rows, 0]
        vc[kvh] = p1["v_cache"][cache_rows, 0]
        q_all = W.to_f64(np.concatenate([f["q_qry"][:, hs], f["q_dec"][:, hs]]))
        kt, vt = O.tail_keys(W.to_f64(np.concatenate([f["k_qry"][:, ks], f["k_dec"][:, ks]])),
                             W.to_f64(np.concatenate([f["v_qry"][:, ks], f["v_dec"][:, ks]])), w.ctx_len, w.rope_theta)
        op, lp = O.phase2_partials(q_all, w.ctx_len, p1["k_cache"], p1["v_cache"], w.block_len, kt, vt, w.ctx_len,
                                   w.rope_theta, w.softmax_scale)
        k_tail[kvh], v_tail[kvh] = kt[:, 0], vt[:, 0]
        opart[:, :, hs] = op
        lpart[:, :, hs] = lp
        del p1, q_ctx, k_ctx, v_ctx
    out, lse = O.merge(opart, lpart)
    qry = {"out": out[:T0], "lse": lse[:T0], "out_part": opart[:, :T0], "lse_part": lpart[:, :T0]}
    dec = [{"out": out[T0 + s:T0 + s + 1], "lse": lse[T0 + s:T0 + s + 1], "out_part": opart[:, T0 + s:T0 + s + 1],
            "lse_part": lpart[:, T0 + s:T0 + s + 1]} for s in range(S)]
    return {"out_ctx": out_ctx, "k_cache": kc, "v_cache": vc, "qry": qry, "dec": dec, "k_tail": k_tail,
            "v_tail": v_tail}


def assert_close(name: str, got: np.ndarray, want: np.ndarray, dtype: str, tol: dict | None = None) -> dict:
    """Compare element by element under the workload's tolerance (or ``tol``,
    {"max": ..., "mean": ... or None}); -inf must match exactly."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{name}: shape {got.shape} != {want.shape}"
    ninf_w, ninf_g = np.isneginf(want), np.isneginf(got)
    assert np.array_equal(ninf_w, ninf_g), f"{name}: -inf pattern differs ({ninf_g.sum()} vs {ninf_w.sum()})"
    assert np.all(np.isfinite(got[~ninf_g])), f"{name}: non-finite values"
    fin = ~ninf_w
    err = np.abs(got[fin] - want[fin])
    mx = float(err.max()) if err.size else 0.0
    mean = float(err.mean()) if err.size else 0.0
    tol = tol or TOL[dtype]
    assert mx <= tol["max"], f"{name}: max abs err {mx:.3e} > {tol['max']:.1e} (mean {mean:.3e})"
    if tol["mean"] is not None:
        assert mean <= tol["mean"], f"{name}: mean abs err {mean:.3e} > {tol['mean']:.1e}"
    return {"max": mx, "mean": mean}


def check_workload(w: W.Workload, seed: int = 0, full_rows: bool | None = None, rows_by_block=None,
                   x: dict | None = None, key_scale: dict | None = None, lse_tol: float | None = None) -> dict:
    """Generate inputs, run GPU and oracle, compare everything; returns error stats.
    ``rows_by_block`` overrides the sampled context rows; ``x`` replaces the
    seeded inputs (same names and layout as ``workloads.all_tensors``);
    ``key_scale`` = {"k_ctx": per context row, "k_tail": per tail row} factors
    the keys were multiplied by: the cached keys are compared after dividing
    both sides by them (a stored key's rounding error scales with the key);
    ``lse_tol`` replaces the maximum error allowed on Phase-2 log-sum-exps."""
    t0 = time.time()
    if x is None:
        x = W.all_tensors(w, seed)
    log(f"{w.name}: inputs ready ({time.time() - t0:.1f}s)")
    if full_rows is None:
        full_rows = w.ctx_len * w.n_q_heads <= 1 << 16
    if rows_by_block is not None:
        cache_rows = np.unique(np.concatenate([(i - 1) * w.block_len + r for i, r in rows_by_block.items()]))
    elif full_rows:
        rows_by_block = {i: np.arange(w.block_len) for i in range(1, w.n_blocks + 1)}
        cache_rows = np.arange(w.ctx_len)
    else:
        rows_by_block = W.sample_rows(w, seed)
        cache_rows = np.unique(np.concatenate([(i - 1) * w.block_len + r for i, r in rows_by_block.items()]))
    gpu = run_gpu(w, x, rows_by_block, cache_rows)
    t1 = time.time()
    ref = run_oracle(w, x, rows_by_block, cache_rows)
    log(f"{w.name}: oracle done ({time.time() - t1:.1f}s)")
    stats = {}
    for i in rows_by_block:
        stats[f"out_ctx[{i}]"] = assert_close(f"{w.name} out_ctx block {i}", gpu.out_ctx[i], ref["out_ctx"][i], w.dtype)
    kc_g, kc_r, kt_g, kt_r = gpu.k_cache, ref["k_cache"], gpu.k_tail, ref["k_tail"]
    if key_scale is not None:
        f = np.asarray(key_scale["k_ctx"], dtype=np.float64)[cache_rows][None, :, None]
        kc_g, kc_r = kc_g / f, kc_r / f
        f = np.asarray(key_scale["k_tail"], dtype=np.float64)[None, :, None]
        kt_g, kt_r = kt_g / f, kt_r / f
    stats["k_cache"] = assert_close(f"{w.name} k_cache", kc_g, kc_r, w.dtype)
    stats["v_cache"] = assert_close(f"{w.name} v_cache", gpu.v_cache, ref["v_cache"], w.dtype)
    stats["k_tail"] = assert_close(f"{w.name} k_tail", kt_g, kt_r, w.dtype)
    stats["v_tail"] = assert_close(f"{w.name} v_tail", gpu.v_tail, ref["v_tail"], w.dtype)
    tol = {k: ({"max": lse_tol, "mean": None} if lse_tol is not None and k.startswith("lse") else None)
           for k in ("out_part", "lse_part", "out", "lse")}
    for key in ("out_part", "lse_part", "out", "lse"):
        stats[f"qry.{key}"] = assert_close(f"{w.name} query {key}", gpu.qry[key], ref["qry"][key], w.dtype, tol[key])
    for s in range(w.n_decode):
        for key in ("out_part", "lse_part", "out", "lse"):
            stats[f"dec{s}.{key}"] = assert_close(f"{w.name} decode {s} {key}", gpu.dec[s][key], ref["dec"][s][key],
                                                  w.dtype, tol[key])
    worst = max(v["max"] for v in stats.values())
    log(f"{w.name}: PASS (worst max abs err {worst:.3e})")
    return stats
