/*
 * starattn.h - C ABI of libstarattn, the Star Attention two-phase attention hot
 * path for one MI355X (gfx950) GPU.
 *
 * The operations follow "Star Attention 完全拆解(一)" (page 1 of the Star
 * Attention pages):
 *   - "Phase 1: augmented context" and "local attention and KV discard":
 *     the context c = [c_1 .. c_n] of n blocks of b tokens; every block c_i
 *     (i > 1) attends causally to itself and to a prepended copy of the anchor
 *     block c_1, the anchor at positions [0, A), block i at [(i-1)b, ib); only
 *     the non-anchor KV is kept.
 *   - "Phase 2: local attention and local statistics", "assembling the global
 *     result" and "numerical stability: log-sum-exp": query and generated
 *     tokens attend to each host's KV, every host returns a normalised local
 *     output A_h and its log-sum-exp, and the partials merge exactly.
 *   - "query-host logic": the KV of query and generated tokens lives only on
 *     the query host (the last host); here it is a separate tail partition.
 * On one GPU the pages' hosts become partitions of one KV cache.
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers owned by the caller (the one
 *     host array is anchor_pos of sa_phase1_encode_anchor_at); the library
 *     allocates nothing, keeps no state between calls (the one exception is the
 *     fixed device array of sa_phase2_step_noalloc) and borrows pointers for
 *     the stream-ordered lifetime of the call. Outputs must not alias inputs.
 *   - Every tensor is dense, row-major, in the element type `desc->dtype`
 *     (float32 or bfloat16), unless a float32 type is stated; every pointer
 *     must be 16-byte aligned.
 *   - Layouts: Q-like tensors are [tokens][n_q_heads][head_dim], K/V inputs
 *     are [tokens][n_kv_heads][head_dim] (pre-RoPE K), caches are
 *     [n_kv_heads][rows][head_dim] holding RoPE'd K and plain V.
 *   - RoPE pairs element j with j + head_dim/2 and rotates it by
 *     pos * rope_theta^(-2j/head_dim) radians (no frequency scaling). Query
 *     head h reads KV head h / (n_q_heads / n_kv_heads).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and deterministic (fixed reduction order).
 *   - Return value: SA_OK, or a negative error code; no call aborts or throws.
 *     On error nothing was launched and sa_last_error() describes the cause.
 *     Argument checks happen before any launch (only device queries precede
 *     them).
 */
#ifndef STARATTN_H
#define STARATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 1

enum {
  SA_OK = 0,
  SA_EINVAL = -1,     /* null/misaligned pointer, inconsistent sizes, overflow of the tail */
  SA_ENOTSUP = -2,    /* head_dim / dtype combination not implemented */
  SA_EWORKSPACE = -3, /* workspace smaller than sa_workspace_bytes() */
  SA_EHIP = -4        /* HIP launch/runtime error (message from hipGetErrorString) */
};

typedef enum { SA_F32 = 0, SA_BF16 = 1 } sa_dtype;

typedef struct sa_attn_desc {
  int32_t n_q_heads;     /* Hq >= 1 */
  int32_t n_kv_heads;    /* Hkv >= 1, Hq % Hkv == 0 (GQA) */
  int32_t head_dim;      /* d: 64 or 128 */
  int32_t dtype;         /* sa_dtype of Q, K, V, caches and the Phase-1 output */
  double rope_theta;     /* RoPE base, > 0 */
  float softmax_scale;   /* scores are softmax_scale * q.k (the pages use 1/sqrt(d)) */
  int32_t reserved;      /* must be 0 */
} sa_attn_desc;

enum { SA_CALL_PHASE1 = 1, SA_CALL_PHASE2 = 2 };

/*
 * Phase 1, context encoding (page 1, "Phase 1: augmented context" eq. for c',
 * "local attention and KV discard", and the blockwise-context code excerpt).
 *
 * ctx_len   L, a multiple of block_len, at most 2^30 (as is every tail_cap: the
 *           kernels index cache rows in 32 bits).  block_len b >= 1.
 *           anchor_len A in [1, b] (the first A tokens of c_1 are the anchor).
 * q_ctx     [L][Hq][d]  pre-RoPE queries of the context tokens.
 * k_ctx     [L][Hkv][d] pre-RoPE keys.   v_ctx [L][Hkv][d] values.
 * out_ctx   [L][Hq][d]  written: attention output of every context token. Block 1
 *           attends causally to itself; block i > 1 attends to all anchor tokens
 *           and causally to its own tokens (positions as above).
 * k_cache   [Hkv][L][d] written: RoPE'd keys at their true positions.
 * v_cache   [Hkv][L][d] written: values. Only the L real rows are cached; no
 *           per-block anchor copy exists.
 * workspace optional device memory, 16-byte aligned. With at least
 *           sa_workspace_bytes(SA_CALL_PHASE1, ...) bytes (256) the bf16 kernel
 *           hands its jobs out at run time: each XCD first takes its own share
 *           and then the next jobs of the XCD furthest behind, so the faster
 *           XCDs are not left idle at the end. With NULL (or fewer bytes) the
 *           jobs keep a static order. The outputs are the same, bit for bit,
 *           either way. Its contents on entry do not matter; concurrent calls
 *           must not share one workspace.
 */
int sa_phase1_encode(const sa_attn_desc* desc, int64_t ctx_len, int64_t block_len, int64_t anchor_len,
                     const void* q_ctx, const void* k_ctx, const void* v_ctx,
                     void* out_ctx, void* k_cache, void* v_cache,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Anchor block choices of sa_phase1_encode_anchor. */
enum { SA_ANCHOR_FIRST = 0, SA_ANCHOR_PREVIOUS = 1 };

/*
 * Phase 1 with a choice of anchor block (page 1, section on vLLM's chunked
 * local attention backend, which recounts the paper's ablation that used the
 * block right before the current one as anchor instead of the first block).
 *
 * anchor_kind  SA_ANCHOR_FIRST: exactly sa_phase1_encode (the anchor is the
 *              first A tokens of c_1, at positions [0, A)).
 *              SA_ANCHOR_PREVIOUS: block i > 1 attends to the first A tokens of
 *              c_{i-1}, at their own positions [(i-2)b, (i-2)b + A), and
 *              causally to itself; for i = 2 both choices are the same.
 * All other arguments, the outputs (the KV cache does not depend on the anchor)
 * and the errors are those of sa_phase1_encode; an unknown anchor_kind is
 * SA_EINVAL.
 */
int sa_phase1_encode_anchor(const sa_attn_desc* desc, int64_t ctx_len, int64_t block_len, int64_t anchor_len,
                            int32_t anchor_kind, const void* q_ctx, const void* k_ctx, const void* v_ctx,
                            void* out_ctx, void* k_cache, void* v_cache,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * Phase 1 with the anchor at other position IDs (page 3, section 4.1 on the
 * anchor block's position and content: the paper's ablation gave the anchor
 * random position IDs, or IDs in line with the context block, and found the
 * accuracy barely changed; page 1, "scope and engineering notes", has the IDs
 * drawn from the prefix).
 *
 * anchor_pos  host array of L/b int64 entries, read during the call only.
 *             Entry i - 1 is the position ID of the first anchor token in the
 *             augmented block of block i > 1: the anchor (the first A tokens of
 *             c_1) sits at anchor_pos[i-1] + [0, A), block i keeps [(i-1)b, ib).
 *             Each entry i - 1 >= 1 must lie in [0, (i-1)b - A] (the anchor
 *             inside the prefix); all zeros is sa_phase1_encode, (i-1)b - A
 *             places the anchor right before the block. Entry 0 is ignored.
 * workspace   device memory, 16-byte aligned: the anchor's keys rotated for
 *             every block i > 1 ([Hkv][L/b - 1][A][d] in the desc dtype) from
 *             its start, padded to 256 bytes, then optionally the 256 bytes of
 *             the run-time job order (as in sa_phase1_encode).
 *             sa_anchor_at_workspace_bytes(...) gives both; the keys alone
 *             are required. Its contents on entry do not matter; it must stay
 *             untouched until the call's work on `stream` is done. May be NULL
 *             when n = 1 (the job order then static).
 * Everything else is as in sa_phase1_encode; the KV cache holds the true
 * positions either way. Errors: SA_EINVAL for a NULL anchor_pos or an entry
 * out of range, SA_EWORKSPACE for a short workspace, else as sa_phase1_encode.
 */
int sa_phase1_encode_anchor_at(const sa_attn_desc* desc, int64_t ctx_len, int64_t block_len, int64_t anchor_len,
                               const int64_t* anchor_pos, const void* q_ctx, const void* k_ctx, const void* v_ctx,
                               void* out_ctx, void* k_cache, void* v_cache,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of sa_phase1_encode_anchor_at: (L/b - 1) * A * Hkv * d *
 * element size (the rotated keys, required) rounded up to 256, plus 256 for the
 * run-time job order; 0 for invalid arguments. */
size_t sa_anchor_at_workspace_bytes(const sa_attn_desc* desc, int64_t ctx_len, int64_t block_len,
                                    int64_t anchor_len);

/*
 * Append KV of query or generated tokens to the query host's tail (page 1,
 * "query-host logic": only the last host adds new tokens' KV; Phase 2 query
 * positions continue at L).
 *
 * k_new, v_new  [t_new][Hkv][d] pre-RoPE keys and values of the new tokens.
 * pos0          position of the first new token (L for the query step).
 * k_tail, v_tail [Hkv][tail_cap][d]; rows [tail_len, tail_len + t_new) are written,
 *               K RoPE'd at pos0 + r. Requires tail_len + t_new <= tail_cap.
 * t_new == 0 is a no-op.
 */
int sa_decode_append(const sa_attn_desc* desc, const void* k_new, const void* v_new,
                     int64_t t_new, int64_t pos0, void* k_tail, void* v_tail,
                     int64_t tail_cap, int64_t tail_len, void* stream);

/*
 * Phase 2 local attention of every partition (page 1, "Phase 2: local attention
 * and local statistics", eq. for A_h and s_h, in the LSE form of "numerical
 * stability: log-sum-exp").
 *
 * q         [t_q][Hq][d] pre-RoPE query rows; token t sits at position q_pos0 + t.
 * k_cache/v_cache  the Phase-1 cache [Hkv][ctx_len][d]; context partition j (1..n,
 *           n = ctx_len / block_len) is rows [(j-1)b, jb) at positions equal to the row.
 * k_tail/v_tail    [Hkv][tail_cap][d]; the tail partition (index n) holds rows
 *           [0, tail_len) at positions tail_pos0 + r. tail_len may be 0.
 * A key is visible to a query row iff key position <= query position.
 * out_part  float32 [n+1][t_q][Hq][d]: A_j, softmax over partition j's visible keys
 *           times V (0 if the partition has no visible key).
 * lse_part  float32 [n+1][t_q][Hq]: natural log of sum exp(softmax_scale * q.k) over
 *           the visible keys (-inf if none).
 * workspace device scratch of at least sa_workspace_bytes(SA_CALL_PHASE2, ...) bytes
 *           with the same (ctx_len, block_len, t_q, tail_cap) on the same device;
 *           its contents before the call do not matter. Calls that may run at the
 *           same time must not share a workspace.
 */
int sa_phase2_partial(const sa_attn_desc* desc, const void* q, int64_t t_q, int64_t q_pos0,
                      const void* k_cache, const void* v_cache, int64_t ctx_len, int64_t block_len,
                      const void* k_tail, const void* v_tail, int64_t tail_cap, int64_t tail_len,
                      int64_t tail_pos0, float* out_part, float* lse_part,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Global merge of the partials (page 1, "assembling the global result":
 * s_global = sum_h s_h, A_global = sum_h (s_h / s_global) A_h; evaluated with the
 * largest lse subtracted first, as "numerical stability: log-sum-exp" advises).
 *
 * out_part [n_parts][t_q][n_q_heads][head_dim] and lse_part [n_parts][t_q][n_q_heads],
 *          float32. Partitions with lse = -inf get weight 0.
 * out      [t_q][n_q_heads][head_dim] in out_dtype (sa_dtype).
 * lse      float32 [t_q][n_q_heads] or NULL. Rows with no visible key anywhere get
 *          out = 0 and lse = -inf.
 */
int sa_phase2_merge(int32_t n_parts, int64_t t_q, int32_t n_q_heads, int32_t head_dim,
                    const float* out_part, const float* lse_part, void* out, int32_t out_dtype,
                    float* lse, void* stream);

/*
 * One whole Phase-2 step on the query host in one call (page 1, "query-host
 * logic" for the append, "Phase 2: local attention and local statistics" and
 * "assembling the global result" for the rest): sa_decode_append of the t new
 * tokens, then local attention of every partition and the global merge, with
 * the split-KV chunks of every partition merged straight into `out` (one merge
 * launch instead of a chunk merge and a partition merge; no out_part/lse_part
 * buffers). For decode-shaped steps (bf16, at most 8 query rows per KV head) the
 * partial kernel's tail workgroups write the new rows themselves, so the step
 * is two launches.
 *
 * Positions follow the pages' sequence: tail row r sits at position ctx_len + r,
 * so the new tokens take positions ctx_len + tail_len ... and their queries the
 * same positions.
 * q             [t][Hq][d] pre-RoPE queries of the new tokens (t >= 1).
 * k_new, v_new  [t][Hkv][d] pre-RoPE keys and values of the new tokens.
 * k_cache/v_cache  the Phase-1 cache [Hkv][ctx_len][d].
 * k_tail/v_tail [Hkv][tail_cap][d]; rows [0, tail_len) are present, rows
 *               [tail_len, tail_len + t) are written. Requires tail_len + t <= tail_cap.
 * out           [t][Hq][d] in desc->dtype: attention of each new token over the
 *               context and the tail rows up to itself.
 * lse           float32 [t][Hq] or NULL.
 * workspace     at least sa_workspace_bytes(SA_CALL_PHASE2, desc, ctx_len,
 *               block_len, t, tail_cap) bytes (as for sa_phase2_partial).
 * The result equals sa_decode_append + sa_phase2_partial + sa_phase2_merge up to
 * rounding: the merge order, and for query steps the bf16 rounding of the
 * rotated queries (the step's append kernel rotates them with the library
 * sine/cosine, sa_phase2_partial's tile kernel with the hardware one).
 */
int sa_phase2_step(const sa_attn_desc* desc, const void* q, const void* k_new, const void* v_new, int64_t t,
                   const void* k_cache, const void* v_cache, int64_t ctx_len, int64_t block_len,
                   void* k_tail, void* v_tail, int64_t tail_cap, int64_t tail_len,
                   void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * sa_phase2_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, checks, kernels and
 * results as sa_phase2_step (bit for bit); its split-KV chunk partials go to a
 * fixed array of SA_NOALLOC_SCRATCH_BYTES bytes that the library holds on each
 * GPU it runs on from load until the process ends. It calls no allocator.
 *
 * A step whose sa_workspace_bytes(SA_CALL_PHASE2, ...) exceeds
 * SA_NOALLOC_SCRATCH_BYTES returns SA_EWORKSPACE (every query and decode step
 * of the Llama-3.1-8B/70B-shaped layers up to 1M context fits). The array of
 * the current device is used, so `stream` must belong to the current device.
 * Every such call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (other streams, other threads) race and must not be issued;
 * calls ordered on one stream are safe. Nothing in the array needs to start
 * at zero.
 */
#define SA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int sa_phase2_step_noalloc(const sa_attn_desc* desc, const void* q, const void* k_new, const void* v_new, int64_t t,
                           const void* k_cache, const void* v_cache, int64_t ctx_len, int64_t block_len,
                           void* k_tail, void* v_tail, int64_t tail_cap, int64_t tail_len,
                           void* out, float* lse, void* stream);

/*
 * Decode steps of several sequences in one call (up to SA_MAX_BATCH), for
 * serving many requests at once: for each sequence exactly sa_phase2_step with
 * one new token, up to the rounding of the merge order. Every sequence has its
 * own context cache, tail and lengths; all share `desc`.
 *
 * Implemented for bf16 with at most 8 query heads per KV head (other
 * descriptors: SA_ENOTSUP). Two launches in all, whatever n_seq: the split-KV
 * partials of every sequence's partitions, whose tail workgroups also append the
 * new rows (one chunk length for the whole batch, so the grid fills the GPU),
 * and the merges.
 * Sequences must not share tails or outputs.
 */
#define SA_MAX_BATCH 16
typedef struct sa_decode_seq {
  const void* q;         /* [Hq][d] pre-RoPE query of the new token */
  const void* k_new;     /* [Hkv][d] pre-RoPE key of the new token */
  const void* v_new;     /* [Hkv][d] its value */
  const void* k_cache;   /* [Hkv][ctx_len][d] Phase-1 cache (RoPE'd K) */
  const void* v_cache;   /* [Hkv][ctx_len][d] */
  void* k_tail;          /* [Hkv][tail_cap][d]; row tail_len is written */
  void* v_tail;
  void* out;             /* [Hq][d] in desc->dtype */
  float* lse;            /* [Hq] float32, or NULL */
  int64_t ctx_len;       /* L, a multiple of block_len, at most 2^30 */
  int64_t block_len;
  int64_t tail_cap;      /* at most 2^30 */
  int64_t tail_len;      /* tail rows before the step; requires tail_len + 1 <= tail_cap */
} sa_decode_seq;

/* Workspace bytes of sa_decode_step_batched for these sequences (it depends on
 * their ctx_len, block_len and tail_cap, not on tail_len); 0 if invalid. */
size_t sa_decode_batch_workspace_bytes(const sa_attn_desc* desc, int32_t n_seq, const sa_decode_seq* seqs);
int sa_decode_step_batched(const sa_attn_desc* desc, int32_t n_seq, const sa_decode_seq* seqs,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace bytes a call needs for these sizes (0 = none). Returns 0 for
 * invalid arguments as well; the call itself reports the error. */
size_t sa_workspace_bytes(int32_t which_call, const sa_attn_desc* desc, int64_t ctx_len,
                          int64_t block_len, int64_t t_q, int64_t tail_cap);

/*
 * Machine ceilings (measurement utilities, not part of the attention path).
 * The caller times them (e.g. with HIP events on `stream`).
 *
 * sa_calibrate_stream_read: reads `bytes` (a multiple of 16) of device memory at
 *   `buf` once with 16-byte loads; `sink` is a device buffer of >= 16 bytes that
 *   the kernel may write.
 * sa_calibrate_mfma: n_workgroups x 4 wavefronts each run `iters` x 8 independent
 *   v_mfma_f32_32x32x16_bf16 (32768 FLOP each), no memory traffic; `sink` is a
 *   device buffer of >= 1024 bytes that the kernel may write.
 */
int sa_calibrate_stream_read(const void* buf, size_t bytes, void* sink, void* stream);
int sa_calibrate_mfma(int32_t iters, int32_t n_workgroups, void* sink, void* stream);

/*
 * The current device's properties that the vendor peaks derive from (a
 * measurement utility): compute units, peak shader clock and memory clock in
 * kHz, and memory bus width in bits (host pointers, each written; none may be
 * NULL). The dense bf16 MFMA peak is n_cus x clock x 4096 FLOP per clock on
 * CDNA4; the HBM3E peak is 4 x mem_clock x bus_width / 8 bytes per second (four
 * transfers per pin per reported memory clock: MI355X reports 2000 MHz for its
 * 8 Gb/s pins). SA_EHIP when the runtime cannot tell.
 */
int sa_device_info(int32_t* n_cus, int32_t* clock_khz, int32_t* mem_clock_khz, int32_t* mem_bus_bits);

/* Description of the calling thread's last error ("" if none). */
const char* sa_last_error(void);

/* SA_ABI_VERSION of the loaded library. */
int32_t sa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* STARATTN_H */
