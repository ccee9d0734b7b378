"""Seeded synthetic workloads for the Star Attention hot path.

This module only describes shapes and draws the input tensors. It holds none of
the method's arithmetic (no RoPE, no attention, no merge), so that both the
fp64 oracle and the HIP path can consume exactly the same bits.

Workload shapes follow the Star Attention pages: Llama-3.1 8B / 70B attention
layer shapes (page 1, "cost of long context": 8 KV heads, head_dim 128, bf16),
context split into n blocks of b tokens with the first block as anchor (page 1,
"problem definition"), and the long-context + short-query regime (page 1, "the
two phases"). Real activations need trained weights, which are not available;
Q/K/V rows are i.i.d. N(0,1) instead, with the keys of positions 0..3 shifted by
3 along one seeded unit direction so that an attention-sink-like structure sits
inside the anchor block.

Generation recipe (identical for every consumer):
  * every tensor is drawn in chunks of ``CHUNK_ROWS`` rows; chunk ``c`` of tensor
    ``t`` uses ``numpy.random.Generator(PCG64(SeedSequence([seed, config_id, t, c])))``
    and ``standard_normal(dtype=float32)`` of shape ``[rows, heads, head_dim]``;
  * the sink direction is ``u = z/|z|`` with ``z`` the float64 standard normal
    vector of tensor id ``T_SINK``; context keys at positions 0..3 get ``+3u``
    added in float32 (all KV heads), before any rounding;
  * bf16 workloads round the float32 values to bfloat16 with round-to-nearest-even
    and hand out the raw 16-bit patterns (``numpy.uint16``).
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK_ROWS = 4096

# tensor ids (part of the seed key)
T_Q_CTX, T_K_CTX, T_V_CTX = 0, 1, 2
T_Q_QRY, T_K_QRY, T_V_QRY = 3, 4, 5
T_Q_DEC, T_K_DEC, T_V_DEC = 6, 7, 8
T_SINK = 9
T_ANCHOR_POS = 10

SINK_POSITIONS = 4
SINK_SHIFT = 3.0


@dataclasses.dataclass(frozen=True)
class Workload:
    """One attention layer's Star Attention workload."""

    name: str
    config_id: int
    dtype: str            # "f32" or "bf16"
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx_len: int          # L
    block_len: int        # b
    anchor_len: int       # A (1..b)
    n_query: int          # T0 query tokens
    n_decode: int         # S decode steps (one row each)
    rope_theta: float
    sink: bool
    anchor: str = "first"  # anchor block: "first" (c_1, the method) or "previous" (c_{i-1}, an ablation)
    anchor_at: str = "own"  # anchor position IDs: "own", "random" (from the prefix) or "adjacent" (right before c_i)

    @property
    def n_blocks(self) -> int:
        return self.ctx_len // self.block_len

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def softmax_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def tail_cap(self) -> int:
        return self.n_query + self.n_decode

    def with_block(self, block_len: int, anchor_len: int | None = None) -> "Workload":
        a = block_len if anchor_len is None else anchor_len
        return dataclasses.replace(self, name=f"{self.name.split('@')[0]}@b{block_len}",
                                   block_len=block_len, anchor_len=a)

    def with_anchor(self, anchor: str) -> "Workload":
        """The same inputs with another anchor block (the seed key does not change)."""
        return dataclasses.replace(self, name=f"{self.name}+{anchor}", anchor=anchor)

    def with_anchor_at(self, anchor_at: str) -> "Workload":
        """The same inputs with the anchor at other position IDs (see ``anchor_positions``)."""
        assert anchor_at in ANCHOR_AT, anchor_at
        return dataclasses.replace(self, name=f"{self.name}+anchor_{anchor_at}", anchor_at=anchor_at)


ANCHOR_AT = ("own", "random", "adjacent")


def anchor_positions(w: Workload, seed: int = 0) -> np.ndarray | None:
    """First position ID of the anchor in each augmented block (int64 [n], entry
    i - 1 for block i; entry 0, block 1, has no anchor and is 0), or None when the
    anchor keeps its own positions. These are inputs like the tensors:
      * "random": for block i >= 2 an integer drawn uniformly from
        [0, (i - 1) b - A] (the anchor lands somewhere inside the prefix), from
        ``Generator(PCG64(SeedSequence([seed, config_id, T_ANCHOR_POS, 0])))``;
      * "adjacent": (i - 1) b - A, the positions right before block i.
    """
    if w.anchor_at == "own":
        return None
    n, b, A = w.n_blocks, w.block_len, w.anchor_len
    hi = np.array([(i - 1) * b - A for i in range(1, n + 1)], dtype=np.int64)
    hi[0] = 0
    if w.anchor_at == "adjacent":
        return hi
    assert w.anchor_at == "random", w.anchor_at
    pos = _rng(seed, w, T_ANCHOR_POS, 0).integers(0, hi + 1, dtype=np.int64)
    pos[0] = 0
    return pos


# The five workloads of the Star Attention hot path (ids are part of the seed key).
SMALL_F32 = Workload("small_f32_2k", 1, "f32", 4, 1, 64, 2048, 512, 512, 16, 8, 1.0e4, False)
LLAMA8B_32K = Workload("llama8b_32k", 2, "bf16", 32, 8, 128, 32768, 8192, 8192, 64, 32, 5.0e5, True)
LLAMA8B_128K = Workload("llama8b_128k", 3, "bf16", 32, 8, 128, 131072, 32768, 32768, 64, 32, 5.0e5, True)
LLAMA70B_128K = Workload("llama70b_128k", 4, "bf16", 64, 8, 128, 131072, 32768, 32768, 128, 64, 5.0e5, True)
LLAMA8B_1M = Workload("llama8b_1m", 5, "bf16", 32, 8, 128, 1048576, 65536, 65536, 64, 16, 5.0e5, True)

LLAMA8B_128K_SWEEP = tuple(LLAMA8B_128K.with_block(b) for b in (4096, 8192, 16384, 32768))

WORKLOADS = {w.name: w for w in (SMALL_F32, LLAMA8B_32K, LLAMA8B_128K, LLAMA70B_128K, LLAMA8B_1M)}


def _rows_and_heads(w: Workload, tensor_id: int) -> tuple[int, int]:
    rows = {T_Q_CTX: w.ctx_len, T_K_CTX: w.ctx_len, T_V_CTX: w.ctx_len,
            T_Q_QRY: w.n_query, T_K_QRY: w.n_query, T_V_QRY: w.n_query,
            T_Q_DEC: w.n_decode, T_K_DEC: w.n_decode, T_V_DEC: w.n_decode}[tensor_id]
    heads = w.n_q_heads if tensor_id in (T_Q_CTX, T_Q_QRY, T_Q_DEC) else w.n_kv_heads
    return rows, heads


def _rng(seed: int, w: Workload, tensor_id: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, w.config_id, tensor_id, chunk])))


def sink_direction(w: Workload, seed: int = 0) -> np.ndarray:
    """Unit vector (float64, [head_dim]) along which the first context keys are shifted."""
    z = _rng(seed, w, T_SINK, 0).standard_normal(w.head_dim)
    return z / np.linalg.norm(z)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_f64(x: np.ndarray) -> np.ndarray:
    """Widen a workload tensor (float32 or bf16 bit patterns) to float64."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def _chunk(w: Workload, tensor_id: int, seed: int, c: int, rows: int, heads: int) -> np.ndarray:
    r0 = c * CHUNK_ROWS
    n = min(CHUNK_ROWS, rows - r0)
    x = _rng(seed, w, tensor_id, c).standard_normal((n, heads, w.head_dim), dtype=np.float32)
    if tensor_id == T_K_CTX and w.sink and r0 < SINK_POSITIONS:
        u = (SINK_SHIFT * sink_direction(w, seed)).astype(np.float32)
        x[: min(SINK_POSITIONS - r0, n)] += u
    if w.dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def tensor(w: Workload, tensor_id: int, seed: int = 0, threads: int | None = None) -> np.ndarray:
    """Draw one whole tensor ``[rows, heads, head_dim]`` (float32, or uint16 bf16 bits)."""
    rows, heads = _rows_and_heads(w, tensor_id)
    out = np.empty((rows, heads, w.head_dim), dtype=np.float32 if w.dtype == "f32" else np.uint16)
    n_chunks = (rows + CHUNK_ROWS - 1) // CHUNK_ROWS

    def fill(c: int) -> None:
        r0 = c * CHUNK_ROWS
        out[r0: r0 + CHUNK_ROWS] = _chunk(w, tensor_id, seed, c, rows, heads)

    if n_chunks <= 1:
        for c in range(n_chunks):
            fill(c)
    else:
        n_thr = threads or min(16, len(os.sched_getaffinity(0)))
        with ThreadPoolExecutor(max_workers=n_thr) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out


def all_tensors(w: Workload, seed: int = 0) -> dict[str, np.ndarray]:
    """Every input tensor of one workload, keyed by name."""
    names = {"q_ctx": T_Q_CTX, "k_ctx": T_K_CTX, "v_ctx": T_V_CTX,
             "q_qry": T_Q_QRY, "k_qry": T_K_QRY, "v_qry": T_V_QRY,
             "q_dec": T_Q_DEC, "k_dec": T_K_DEC, "v_dec": T_V_DEC}
    return {k: tensor(w, t, seed) for k, t in names.items()}


def sample_rows(w: Workload, seed: int = 0, n_random: int = 3, span: int | None = None,
                blocks=None) -> dict[int, np.ndarray]:
    """Seeded sample of context rows per block for full-size parity checks.

    Every block contributes rows 0, 1, b/2, b-2, b-1 plus ``n_random`` random rows;
    with ``span``, also one random row in every run of ``span`` consecutive rows
    (so that every tile of that many rows is sampled). ``blocks`` limits the
    blocks (1-based; default all). Returns {block index (1-based): sorted unique
    row offsets inside the block}.
    """
    b = w.block_len
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, w.config_id, 1000, b])))
    out = {}
    for i in range(1, w.n_blocks + 1):
        fixed = [0, 1, b // 2, b - 2, b - 1]
        rnd = rng.integers(0, b, size=n_random).tolist()
        if span:
            starts = np.arange(0, b, span)
            rnd += (starts + rng.integers(0, span, size=len(starts))).tolist()
        if blocks is None or i in blocks:
            out[i] = np.unique(np.clip(np.array(fixed + rnd), 0, b - 1))
    return out
