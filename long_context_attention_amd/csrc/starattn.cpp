// libstarattn C ABI: argument checks, Phase-2 chunk planning and kernel dispatch.
// All argument checks run before any launch, so invalid arguments are reported
// without touching device memory; the only HIP calls made before them are the
// device queries (compute units, occupancy) that size the Phase-2 split.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <string>

#include "../../include/starattn.h"
#include "sa_common.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return SA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Largest context and tail length: the attention kernels keep cache rows in
// 32-bit integers, with room for a tile past the end.
constexpr int64_t kMaxRows = (int64_t)1 << 30;
// Work items of one launch of the one-thread-per-item kernels (RoPE/cache store,
// anchor keys): the grid's total size must stay below 2^32.
constexpr int64_t kMaxLaunchThreads = ((int64_t)1 << 32) - 256;

// a * b for non-negative a, b, saturating at INT64_MAX
int64_t mul_sat(int64_t a, int64_t b) {
  int64_t r;
  return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}

int check_desc(const sa_attn_desc* d) {
  if (!d) return fail(SA_EINVAL, "desc is NULL");
  if (d->n_q_heads < 1 || d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads != 0)
    return fail(SA_EINVAL, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", d->n_q_heads,
                d->n_kv_heads);
  if (d->dtype != SA_F32 && d->dtype != SA_BF16) return fail(SA_EINVAL, "unknown dtype %d", d->dtype);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(SA_ENOTSUP, "head_dim %d not supported (64 or 128)", d->head_dim);
  if (!(d->rope_theta > 0.0) || !isfinite(d->rope_theta))
    return fail(SA_EINVAL, "rope_theta must be positive and finite");
  if (!(d->softmax_scale > 0.f) || !isfinite(d->softmax_scale))
    return fail(SA_EINVAL, "softmax_scale must be positive and finite");
  if (d->reserved != 0) return fail(SA_EINVAL, "desc->reserved must be 0");
  return SA_OK;
}

int check_ptrs(const char* names, int n, const void* const* ptrs) {
  for (int i = 0; i < n; ++i) {
    if (!ptrs[i]) return fail(SA_EINVAL, "pointer #%d of (%s) is NULL", i, names);
    if (!aligned16(ptrs[i])) return fail(SA_EINVAL, "pointer #%d of (%s) is not 16-byte aligned", i, names);
  }
  return SA_OK;
}

int check_blocks(int64_t ctx_len, int64_t block_len) {
  if (ctx_len < 1 || block_len < 1) return fail(SA_EINVAL, "ctx_len and block_len must be >= 1");
  if (ctx_len % block_len != 0)
    return fail(SA_EINVAL, "ctx_len (%lld) must be a multiple of block_len (%lld)", (long long)ctx_len,
                (long long)block_len);
  // the attention kernels index cache rows in 32 bits (with a tile of headroom)
  if (ctx_len > kMaxRows) return fail(SA_EINVAL, "ctx_len (%lld) must be <= 2^30", (long long)ctx_len);
  return SA_OK;
}

sa::RopeTable rope_table(const sa_attn_desc* d) {
  sa::RopeTable t{};
  for (int j = 0; j < d->head_dim / 2; ++j) t.inv_freq[j] = pow(d->rope_theta, -2.0 * j / d->head_dim);
  return t;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SA_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

constexpr float kLog2eF = 1.4426950408889634f;

}  // namespace

namespace sa {

// bf16 decode steps (at most 8 query rows per KV head) take the streaming
// decode kernel, other bf16 steps the MFMA tile kernel (256 rows per tile);
// float32 takes the vector-ALU kernel. Partitions are split
// into chunks so that partitions x chunks x KV heads (x row groups) gives the
// GPU a couple of thousand workgroups.
// Compute units of the current device (cached per device), 0 if unknown.
int64_t device_compute_units() {
  static std::atomic<int> cache[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) return 0;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Workspace of a Phase-2 call: the chunk partials [n_parts][n_chunks][t_q][Hq][d]
// float32, their LSEs, and for the tile kernel the queries rotated and scaled
// (bf16 [t_q][Hq][d]); each part starts on a 256-byte boundary.
P2Layout phase2_ws_layout(const P2Plan& p, int64_t t_q, int32_t n_q_heads, int32_t head_dim) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = (size_t)p.n_parts * p.n_chunks * t_q * n_q_heads;
  P2Layout l{};
  l.lse_off = up(rows * head_dim * sizeof(float));
  l.qrot_off = l.lse_off + up(rows * sizeof(float));
  l.bytes = l.qrot_off + (p.kernel == P2_TILE ? up((size_t)t_q * n_q_heads * head_dim * 2) : 0);
  return l;
}

P2Plan phase2_plan(int64_t ctx_len, int64_t block_len, int64_t t_q, int64_t tail_cap, int32_t n_q_heads,
                   int32_t n_kv_heads, int32_t head_dim, bool bf16) {
  P2Plan p{};
  p.n_parts = (int32_t)(ctx_len / block_len) + 1;
  const int64_t part_len = block_len > tail_cap ? block_len : tail_cap;
  const int64_t rows_per_kv = t_q * (n_q_heads / n_kv_heads);
  const int64_t target = 2048;   // workgroups

  int64_t chunks, align;
  if (bf16 && rows_per_kv <= 8) {
    // Decode: a pure stream over the cache. Every context workgroup gets the
    // same number of keys, and their count fills whole rounds of the resident
    // workgroup slots, so no round runs part-empty. One round, leaving a slot
    // for each KV head's tail workgroup, unless the rows are few (up to 4 per
    // KV head) and a one-round workgroup would stream 0.5 to 4 MiB: there two
    // rounds measured faster (128K, Llama-8B shape: 109 against 113 us;
    // one round wins at 32K, 1M and with 8 rows per KV head). The tail gets
    // only the chunks its rows need (see the launch).
    p.kernel = P2_DECODE;
    const int64_t units = (int64_t)(p.n_parts - 1) * n_kv_heads;
    const int64_t slots = decode_resident_workgroups(head_dim, rows_per_kv);
    if (slots > 0) {
      chunks = (slots - n_kv_heads) / units;
      const int64_t one_round_bytes = (chunks > 0 ? part_len / chunks : part_len) * 2 * head_dim * 2;
      if (rows_per_kv <= 4 && one_round_bytes >= (512 << 10) && one_round_bytes < (4 << 20))
        chunks = (2 * slots + units - 1) / units;
    } else {
      chunks = (1024 + units - 1) / units;
    }
    const int64_t lo = (part_len + 16383) / 16384, hi = (part_len + 127) / 128;
    chunks = chunks < lo ? lo : (chunks > hi ? hi : chunks);
    align = 32;
  } else if (bf16) {
    // Query step: one workgroup per CU (its tiles fill the LDS); the context
    // partitions' chunks fill one round of the CUs (measured best of 1, 2, 4
    // and 8 rounds: 0.19 ms against 0.36 ms at 2048 workgroups for 64 tokens
    // at 128K). More, smaller chunks repeat each workgroup's fixed cost (the
    // RoPE of 256 query rows, 128 KB of fp32 partials written and merged).
    p.kernel = P2_TILE;
    const int64_t row_tiles = (rows_per_kv + 255) / 256;
    const int64_t units = (int64_t)(p.n_parts - 1) * n_kv_heads * row_tiles;
    const int64_t cus = device_compute_units();
    chunks = cus > 0 ? (cus + units - 1) / units : (target + units - 1) / units;
    const int64_t hi = (part_len + 255) / 256;
    chunks = chunks > hi ? hi : chunks;
    align = 64;
  } else {
    // float32: one wavefront per (chunk, query row); chunks of about 128 keys
    // (at most 4096 per partition) keep many wavefronts busy.
    p.kernel = P2_VALU;
    chunks = (part_len + 127) / 128;
    chunks = chunks > 4096 ? 4096 : chunks;
    align = 64;
  }
  if (chunks < 1) chunks = 1;
  int64_t cl = (part_len + chunks - 1) / chunks;
  cl = (cl + align - 1) / align * align;
  p.chunk_len = cl;
  p.n_chunks = (int32_t)((part_len + cl - 1) / cl);
  return p;
}

}  // namespace sa

extern "C" {

int32_t sa_abi_version(void) { return SA_ABI_VERSION; }

const char* sa_last_error(void) { return g_last_error.c_str(); }

size_t sa_workspace_bytes(int32_t which_call, const sa_attn_desc* desc, int64_t ctx_len, int64_t block_len,
                          int64_t t_q, int64_t tail_cap) {
  // Phase 1: the job counters of the run-time job order (optional)
  if (which_call == SA_CALL_PHASE1) return check_desc(desc) == SA_OK ? sa::kPhase1QueueBytes : 0;
  if (which_call != SA_CALL_PHASE2 || check_desc(desc) != SA_OK || check_blocks(ctx_len, block_len) != SA_OK ||
      t_q < 1 || tail_cap < 0)
    return 0;
  const sa::P2Plan p = sa::phase2_plan(ctx_len, block_len, t_q, tail_cap, desc->n_q_heads, desc->n_kv_heads,
                                       desc->head_dim, desc->dtype == SA_BF16);
  return sa::phase2_ws_layout(p, t_q, desc->n_q_heads, desc->head_dim).bytes;
}

int sa_phase1_encode(const sa_attn_desc* desc, int64_t ctx_len, int64_t block_len, int64_t anchor_len,
                     const void* q_ctx, const void* k_ctx, const void* v_ctx, void* out_ctx, void* k_cache,
                     void* v_cache, void* workspace, size_t workspace_bytes, void* stream) {
  return sa_phase1_encode_anchor(desc, ctx_len, block_len, anchor_len, SA_ANCHOR_FIRST, q_ctx, k_ctx, v_ctx, out_ctx,
                                 k_cache, v_cache, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Phase 1 with the anchor block chosen by anchor_prev and, when anchor_pos is
// given, its keys rotated at those position IDs (into the workspace).
int encode(const sa_attn_desc* desc, int64_t ctx_len, int64_t block_len, int64_t anchor_len, bool anchor_prev,
           const int64_t* anchor_pos, const void* q_ctx, const void* k_ctx, const void* v_ctx, void* out_ctx,
           void* k_cache, void* v_cache, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if ((rc = check_blocks(ctx_len, block_len))) return rc;
  if (anchor_len < 1 || anchor_len > block_len)
    return fail(SA_EINVAL, "anchor_len (%lld) must be in [1, block_len]", (long long)anchor_len);
  const void* ptrs[6] = {q_ctx, k_ctx, v_ctx, out_ctx, k_cache, v_cache};
  if ((rc = check_ptrs("q_ctx, k_ctx, v_ctx, out_ctx, k_cache, v_cache", 6, ptrs))) return rc;
  if ((ctx_len + 127) / 128 * desc->n_q_heads > ((int64_t)1 << 31) - 1 ||
      ctx_len * desc->n_kv_heads * (desc->head_dim / 16) > kMaxLaunchThreads)
    return fail(SA_EINVAL, "problem too large for one launch");
  const int64_t n_blocks = ctx_len / block_len;
  const size_t esize = desc->dtype == SA_BF16 ? 2 : 4;
  size_t keys_bytes = 0;   // workspace bytes of the rotated anchor keys (anchor_pos given)
  if (anchor_pos) {
    for (int64_t i = 1; i < n_blocks; ++i)
      if (anchor_pos[i] < 0 || anchor_pos[i] > i * block_len - anchor_len)
        return fail(SA_EINVAL, "anchor_pos[%lld] (%lld) must be in [0, %lld] (the anchor inside the prefix)",
                    (long long)i, (long long)anchor_pos[i], (long long)(i * block_len - anchor_len));
    keys_bytes = (size_t)(n_blocks - 1) * anchor_len * desc->n_kv_heads * desc->head_dim * esize;
    keys_bytes = (keys_bytes + 255) / 256 * 256;
    if (keys_bytes > 0 && !workspace) return fail(SA_EINVAL, "workspace is NULL");
    if (workspace_bytes < keys_bytes)
      return fail(SA_EWORKSPACE, "workspace too small: %zu bytes, need %zu", workspace_bytes, keys_bytes);
  }
  if (workspace && !aligned16(workspace)) return fail(SA_EINVAL, "workspace is not 16-byte aligned");
  // The rest of the workspace, when there is room, holds the job counters of
  // the run-time job order; without it the jobs keep a static order.
  void* queues = workspace && workspace_bytes >= keys_bytes + sa::kPhase1QueueBytes
                     ? static_cast<char*>(workspace) + keys_bytes
                     : nullptr;

  const bool bf16 = desc->dtype == SA_BF16;
  const sa::RopeTable rt = rope_table(desc);
  hipStream_t s = static_cast<hipStream_t>(stream);

  sa::RopeStoreArgs ra{k_ctx, v_ctx, k_cache, v_cache, ctx_len, ctx_len, 0, 0, desc->n_kv_heads, desc->head_dim};
  hipError_t e = sa::launch_rope_store(ra, rt, bf16, s);
  if (e != hipSuccess) return hip_status(e, "rope/cache kernel");
  if (anchor_pos) {
    // the anchor's keys rotated for blocks 2..n, kAnchorPosBatch blocks per launch
    for (int64_t first = 0; first < n_blocks - 1; first += sa::kAnchorPosBatch) {
      sa::AnchorKeysArgs ka{};
      ka.k_src = k_ctx;
      ka.k_dst = workspace;
      ka.anchor_len = anchor_len;
      ka.n_anchors = n_blocks - 1;
      ka.first = first;
      ka.count = (int32_t)(n_blocks - 1 - first < sa::kAnchorPosBatch ? n_blocks - 1 - first : sa::kAnchorPosBatch);
      for (int j = 0; j < ka.count; ++j) ka.pos[j] = anchor_pos[first + 1 + j];
      ka.n_heads = desc->n_kv_heads;
      ka.head_dim = desc->head_dim;
      if ((e = sa::launch_anchor_keys(ka, rt, bf16, s)) != hipSuccess) return hip_status(e, "anchor-keys kernel");
    }
  }

  sa::Phase1Args pa{q_ctx, k_cache, v_cache, out_ctx, ctx_len, block_len, anchor_len,
                    desc->n_q_heads, desc->n_kv_heads, desc->softmax_scale * kLog2eF, anchor_prev ? 1 : 0,
                    anchor_pos && n_blocks > 1 ? workspace : nullptr};
  e = bf16 ? sa::launch_phase1_mfma(pa, rt, desc->head_dim, queues, s)
           : sa::launch_phase1_valu(pa, rt, desc->head_dim, false, s);
  return hip_status(e, "phase-1 attention kernel");
}

}  // namespace

extern "C" {

int sa_phase1_encode_anchor(const sa_attn_desc* desc, int64_t ctx_len, int64_t block_len, int64_t anchor_len,
                            int32_t anchor_kind, const void* q_ctx, const void* k_ctx, const void* v_ctx,
                            void* out_ctx, void* k_cache, void* v_cache, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (anchor_kind != SA_ANCHOR_FIRST && anchor_kind != SA_ANCHOR_PREVIOUS)
    return fail(SA_EINVAL, "unknown anchor_kind %d", (int)anchor_kind);
  return encode(desc, ctx_len, block_len, anchor_len, anchor_kind == SA_ANCHOR_PREVIOUS, nullptr, q_ctx, k_ctx,
                v_ctx, out_ctx, k_cache, v_cache, workspace, workspace_bytes, stream);
}

size_t sa_anchor_at_workspace_bytes(const sa_attn_desc* desc, int64_t ctx_len, int64_t block_len,
                                    int64_t anchor_len) {
  if (check_desc(desc) != SA_OK || check_blocks(ctx_len, block_len) != SA_OK || anchor_len < 1 ||
      anchor_len > block_len)
    return 0;
  const size_t esize = desc->dtype == SA_BF16 ? 2 : 4;
  const size_t keys = (size_t)(ctx_len / block_len - 1) * anchor_len * desc->n_kv_heads * desc->head_dim * esize;
  return (keys + 255) / 256 * 256 + sa::kPhase1QueueBytes;
}

int sa_phase1_encode_anchor_at(const sa_attn_desc* desc, int64_t ctx_len, int64_t block_len, int64_t anchor_len,
                               const int64_t* anchor_pos, const void* q_ctx, const void* k_ctx, const void* v_ctx,
                               void* out_ctx, void* k_cache, void* v_cache, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!anchor_pos) return fail(SA_EINVAL, "anchor_pos is NULL");
  return encode(desc, ctx_len, block_len, anchor_len, false, anchor_pos, q_ctx, k_ctx, v_ctx, out_ctx, k_cache,
                v_cache, workspace, workspace_bytes, stream);
}

int sa_decode_append(const sa_attn_desc* desc, const void* k_new, const void* v_new, int64_t t_new, int64_t pos0,
                     void* k_tail, void* v_tail, int64_t tail_cap, int64_t tail_len, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (t_new < 0 || pos0 < 0 || tail_cap < 0 || tail_len < 0)
    return fail(SA_EINVAL, "t_new, pos0, tail_cap and tail_len must be >= 0");
  if (tail_cap > kMaxRows) return fail(SA_EINVAL, "tail_cap (%lld) must be <= 2^30", (long long)tail_cap);
  if (t_new > tail_cap - tail_len)   // tail_len + t_new > tail_cap, without overflow
    return fail(SA_EINVAL, "tail overflow: tail_len %lld + t_new %lld > tail_cap %lld", (long long)tail_len,
                (long long)t_new, (long long)tail_cap);
  if (t_new == 0) return ok();
  if (t_new * desc->n_kv_heads * (desc->head_dim / 16) > kMaxLaunchThreads)   // t_new <= 2^30: no overflow
    return fail(SA_EINVAL, "problem too large for one launch");
  const void* ptrs[4] = {k_new, v_new, k_tail, v_tail};
  if ((rc = check_ptrs("k_new, v_new, k_tail, v_tail", 4, ptrs))) return rc;
  const sa::RopeTable rt = rope_table(desc);
  sa::RopeStoreArgs ra{k_new, v_new, k_tail, v_tail, t_new, tail_cap, tail_len, pos0, desc->n_kv_heads,
                       desc->head_dim};
  return hip_status(sa::launch_rope_store(ra, rt, desc->dtype == SA_BF16, static_cast<hipStream_t>(stream)),
                    "append kernel");
}

namespace {

// Argument checks shared by sa_phase2_partial and the step calls (all but the
// workspace).
int check_phase2(const sa_attn_desc* desc, int64_t t_q, int64_t q_pos0, const void* q, const void* k_cache,
                 const void* v_cache, int64_t ctx_len, int64_t block_len, const void* k_tail, const void* v_tail,
                 int64_t tail_cap, int64_t tail_len, int64_t tail_pos0) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if ((rc = check_blocks(ctx_len, block_len))) return rc;
  if (t_q < 1 || q_pos0 < 0 || tail_pos0 < 0) return fail(SA_EINVAL, "t_q must be >= 1, positions >= 0");
  if (tail_cap < 0 || tail_len < 0 || tail_len > tail_cap)
    return fail(SA_EINVAL, "tail_len (%lld) must be in [0, tail_cap (%lld)]", (long long)tail_len,
                (long long)tail_cap);
  if (tail_cap > kMaxRows) return fail(SA_EINVAL, "tail_cap (%lld) must be <= 2^30", (long long)tail_cap);
  const void* ptrs[3] = {q, k_cache, v_cache};
  if ((rc = check_ptrs("q, k_cache, v_cache", 3, ptrs))) return rc;
  if (tail_cap > 0) {
    const void* tp[2] = {k_tail, v_tail};
    if ((rc = check_ptrs("k_tail, v_tail", 2, tp))) return rc;
  }
  if (t_q > kMaxRows) return fail(SA_EINVAL, "t_q (%lld) must be <= 2^30", (long long)t_q);
  // every launch of the call (partials, chunk or step merge) stays below 2^32 work items
  const sa::P2Plan p = sa::phase2_plan(ctx_len, block_len, t_q, tail_cap, desc->n_q_heads, desc->n_kv_heads,
                                       desc->head_dim, desc->dtype == SA_BF16);
  const int64_t rows = mul_sat(t_q, desc->n_q_heads);
  const int64_t items = mul_sat(p.n_parts, p.n_chunks);
  int64_t part = 0;
  if (p.kernel == sa::P2_VALU) part = mul_sat(mul_sat(items, rows), 64);
  else if (p.kernel == sa::P2_DECODE) part = mul_sat(mul_sat(items, desc->n_kv_heads), 256);
  else part = mul_sat(mul_sat(mul_sat(items, desc->n_kv_heads), (t_q * (desc->n_q_heads / desc->n_kv_heads) + 255) / 256), 512);
  // chunk merge: up to 256 threads per (partition, row); step merge: up to 512 per row
  const int64_t merge = std::max(mul_sat(mul_sat(p.n_parts, rows), 256), mul_sat(rows, 512));
  if (part > kMaxLaunchThreads || merge > kMaxLaunchThreads)
    return fail(SA_EINVAL, "problem too large for one launch (t_q %lld x %d query heads)", (long long)t_q,
                desc->n_q_heads);
  return SA_OK;
}

// The Phase-2 workspace of a call with checked sizes.
int check_workspace(const sa_attn_desc* desc, int64_t ctx_len, int64_t block_len, int64_t t_q, int64_t tail_cap,
                    const void* workspace, size_t workspace_bytes) {
  const size_t need = sa_workspace_bytes(SA_CALL_PHASE2, desc, ctx_len, block_len, t_q, tail_cap);
  if (workspace_bytes < need || (need && !workspace))
    return fail(SA_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, need);
  if (need && !aligned16(workspace)) return fail(SA_EINVAL, "workspace is not 16-byte aligned");
  return SA_OK;
}

// The split-KV partial kernel: every (partition, chunk) writes its normalised
// output and LSE to the workspace, [n_parts][n_chunks][t_q][Hq]. Fills `ma`
// with the workspace's chunk layout for a merge.
int launch_partials(const sa_attn_desc* desc, const void* q, int64_t t_q, int64_t q_pos0, const void* k_cache,
                    const void* v_cache, int64_t ctx_len, int64_t block_len, const void* k_tail, const void* v_tail,
                    int64_t tail_cap, int64_t tail_len, int64_t tail_pos0, void* workspace, hipStream_t s,
                    sa::P2Plan* plan_out, float** ws_out_p, float** ws_lse_p, const void* k_new = nullptr,
                    const void* v_new = nullptr, int32_t n_new = 0, bool q_rotated = false,
                    int32_t* tail_items_out = nullptr) {
  const sa::P2Plan plan = sa::phase2_plan(ctx_len, block_len, t_q, tail_cap, desc->n_q_heads, desc->n_kv_heads,
                                          desc->head_dim, desc->dtype == SA_BF16);
  const sa::P2Layout lay = sa::phase2_ws_layout(plan, t_q, desc->n_q_heads, desc->head_dim);
  float* ws_out = static_cast<float*>(workspace);
  float* ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + lay.lse_off);
  const bool bf16 = desc->dtype == SA_BF16;
  const sa::RopeTable rt = rope_table(desc);
  // The tile kernel rotates and scales its query rows itself, unless the
  // step's append launch already wrote them rotated into the workspace (then it
  // only loads them). A separate rotation launch measured 5 us slower.
  void* q_rot = plan.kernel == sa::P2_TILE && q_rotated ? static_cast<char*>(workspace) + lay.qrot_off : nullptr;
  sa::Phase2Args pa{q, k_cache, v_cache, k_tail, v_tail, ws_out, ws_lse, t_q, q_pos0, ctx_len, block_len,
                    tail_cap, tail_len, tail_pos0, plan.chunk_len, plan.n_parts - 1, plan.n_chunks,
                    desc->n_q_heads, desc->n_kv_heads, desc->softmax_scale * kLog2eF, 1};
  if (tail_len > plan.chunk_len) pa.n_tail_chunks = (int32_t)((tail_len + plan.chunk_len - 1) / plan.chunk_len);
  if (n_new > 0) {   // an append fused into the decode kernel (the caller checked the plan's kernel)
    pa.k_new = k_new;
    pa.v_new = v_new;
    pa.n_new = n_new;
  }
  pa.q_rot = q_rot;
  // Chunk slots of the tail partition that may hold keys: the decode kernel
  // writes lse = -inf to the others, and so does the tile kernel when the tail
  // rides with a context chunk.
  int32_t tail_items = plan.n_chunks;
  hipError_t e;
  if (plan.kernel == sa::P2_DECODE) {
    e = sa::launch_phase2_decode(pa, rt, desc->head_dim, s);
    tail_items = pa.n_tail_chunks;
  } else if (plan.kernel == sa::P2_TILE) {
    e = sa::launch_phase2_query(pa, rt, desc->head_dim, s, &tail_items);
  } else {
    e = sa::launch_phase2_valu(pa, rt, desc->head_dim, bf16, s);
  }
  if (e != hipSuccess) return hip_status(e, "phase-2 partial kernel");
  if (tail_items_out) *tail_items_out = tail_items;
  *plan_out = plan;
  *ws_out_p = ws_out;
  *ws_lse_p = ws_lse;
  return SA_OK;
}

// Argument checks of a whole step (sa_phase2_step and its no-allocation
// form), all but the workspace.
int check_step(const sa_attn_desc* desc, const void* q, const void* k_new, const void* v_new, int64_t t,
               const void* k_cache, const void* v_cache, int64_t ctx_len, int64_t block_len, const void* k_tail,
               const void* v_tail, int64_t tail_cap, int64_t tail_len, const void* out, const float* lse) {
  int rc = check_phase2(desc, t, ctx_len + tail_len, q, k_cache, v_cache, ctx_len, block_len, k_tail, v_tail,
                        tail_cap, tail_len, ctx_len);
  if (rc) return rc;
  if (t > tail_cap - tail_len)   // tail_len + t > tail_cap, without overflow
    return fail(SA_EINVAL, "tail overflow: tail_len %lld + t %lld > tail_cap %lld", (long long)tail_len,
                (long long)t, (long long)tail_cap);
  if (t * (desc->n_kv_heads + (int64_t)desc->n_q_heads) * (desc->head_dim / 16) > kMaxLaunchThreads)
    return fail(SA_EINVAL, "problem too large for one launch");
  const void* np[3] = {k_new, v_new, out};
  if ((rc = check_ptrs("k_new, v_new, out", 3, np))) return rc;
  if (lse && !aligned16(lse)) return fail(SA_EINVAL, "lse is not 16-byte aligned");
  return SA_OK;
}

// A whole step on checked arguments: the append (unless the decode kernel
// does it), the partials, and one merge of every (partition, chunk) item.
int run_step(const sa_attn_desc* desc, const void* q, const void* k_new, const void* v_new, int64_t t,
             const void* k_cache, const void* v_cache, int64_t ctx_len, int64_t block_len, void* k_tail, void* v_tail,
             int64_t tail_cap, int64_t tail_len, void* out, float* lse, void* workspace, hipStream_t s) {
  const int64_t pos0 = ctx_len + tail_len;
  // The decode kernel appends the new rows itself; the other kernels need the
  // append first.
  const sa::P2Plan plan0 = sa::phase2_plan(ctx_len, block_len, t, tail_cap, desc->n_q_heads, desc->n_kv_heads,
                                           desc->head_dim, desc->dtype == SA_BF16);
  const bool fused_append = plan0.kernel == sa::P2_DECODE;
  // For the tile kernel the append kernel also rotates the new tokens' queries
  // (the same positions) into the workspace.
  const bool rot_q = plan0.kernel == sa::P2_TILE;
  if (!fused_append) {
    const sa::RopeTable rt = rope_table(desc);
    sa::RopeStoreArgs ra{k_new, v_new, k_tail, v_tail, t, tail_cap, tail_len, pos0, desc->n_kv_heads,
                         desc->head_dim};
    if (rot_q) {
      ra.q_src = q;
      ra.q_dst = static_cast<char*>(workspace) +
                 sa::phase2_ws_layout(plan0, t, desc->n_q_heads, desc->head_dim).qrot_off;
      ra.q_heads = desc->n_q_heads;
      ra.q_scale = desc->softmax_scale * kLog2eF;
    }
    hipError_t e = sa::launch_rope_store(ra, rt, desc->dtype == SA_BF16, s);
    if (e != hipSuccess) return hip_status(e, "append kernel");
  }
  sa::P2Plan plan;
  float *ws_out, *ws_lse;
  int32_t tail_items = 0;
  int rc = launch_partials(desc, q, t, pos0, k_cache, v_cache, ctx_len, block_len, k_tail, v_tail, tail_cap,
                           tail_len + t, ctx_len, workspace, s, &plan, &ws_out, &ws_lse, k_new, v_new,
                           fused_append ? (int32_t)t : 0, rot_q, &tail_items);
  if (rc) return rc;
  // every (partition, chunk) item of a row -> the output, in one launch; the
  // tail partition's trailing slots that hold no key (lse = -inf) are left out
  sa::MergeArgs ma{ws_out, ws_lse, out, lse, (int64_t)(plan.n_parts - 1) * plan.n_chunks + tail_items,
                   t * desc->n_q_heads, 1, desc->head_dim};
  return hip_status(sa::launch_merge(ma, desc->dtype == SA_BF16, s), "phase-2 merge kernel");
}

// The no-allocation step's workspace: one array per GPU in the code object,
// resident from library load to process exit. Every no-allocation call on a
// GPU uses that GPU's copy, so such calls must not overlap on one GPU; no part
// of it needs to start at zero (every byte a call reads, the same call wrote).
// Host code never passes the array's name to a kernel (on the host it is only
// a stand-in): scratch_address() gives the device address.
constexpr size_t kScratchBytes = SA_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];   // device address of `scratch`, per device, once looked up

// The current device's address of `scratch`, looked up once per device (with
// that device current).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SA_EHIP, "device %d is beyond the %d devices the no-allocation step serves", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(SA_EHIP, "hipGetSymbolAddress(scratch) gave a null address");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return SA_OK;
}

}  // namespace

int sa_phase2_partial(const sa_attn_desc* desc, const void* q, int64_t t_q, int64_t q_pos0, const void* k_cache,
                      const void* v_cache, int64_t ctx_len, int64_t block_len, const void* k_tail,
                      const void* v_tail, int64_t tail_cap, int64_t tail_len, int64_t tail_pos0, float* out_part,
                      float* lse_part, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_phase2(desc, t_q, q_pos0, q, k_cache, v_cache, ctx_len, block_len, k_tail, v_tail, tail_cap,
                        tail_len, tail_pos0);
  if (rc) return rc;
  if ((rc = check_workspace(desc, ctx_len, block_len, t_q, tail_cap, workspace, workspace_bytes))) return rc;
  const void* op[2] = {out_part, lse_part};
  if ((rc = check_ptrs("out_part, lse_part", 2, op))) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  sa::P2Plan plan;
  float *ws_out, *ws_lse;
  if ((rc = launch_partials(desc, q, t_q, q_pos0, k_cache, v_cache, ctx_len, block_len, k_tail, v_tail, tail_cap,
                            tail_len, tail_pos0, workspace, s, &plan, &ws_out, &ws_lse)))
    return rc;
  // chunks -> per-partition partials
  sa::MergeArgs ma{ws_out, ws_lse, out_part, lse_part, plan.n_chunks, t_q * desc->n_q_heads, plan.n_parts,
                   desc->head_dim};
  return hip_status(sa::launch_merge(ma, false, s), "phase-2 chunk merge kernel");
}

int sa_phase2_step(const sa_attn_desc* desc, const void* q, const void* k_new, const void* v_new, int64_t t,
                   const void* k_cache, const void* v_cache, int64_t ctx_len, int64_t block_len, void* k_tail,
                   void* v_tail, int64_t tail_cap, int64_t tail_len, void* out, float* lse, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int rc = check_step(desc, q, k_new, v_new, t, k_cache, v_cache, ctx_len, block_len, k_tail, v_tail, tail_cap,
                      tail_len, out, lse);
  if (rc) return rc;
  if ((rc = check_workspace(desc, ctx_len, block_len, t, tail_cap, workspace, workspace_bytes))) return rc;
  return run_step(desc, q, k_new, v_new, t, k_cache, v_cache, ctx_len, block_len, k_tail, v_tail, tail_cap, tail_len,
                  out, lse, workspace, static_cast<hipStream_t>(stream));
}

int sa_phase2_step_noalloc(const sa_attn_desc* desc, const void* q, const void* k_new, const void* v_new, int64_t t,
                           const void* k_cache, const void* v_cache, int64_t ctx_len, int64_t block_len,
                           void* k_tail, void* v_tail, int64_t tail_cap, int64_t tail_len, void* out, float* lse,
                           void* stream) {
  int rc = check_step(desc, q, k_new, v_new, t, k_cache, v_cache, ctx_len, block_len, k_tail, v_tail, tail_cap,
                      tail_len, out, lse);
  if (rc) return rc;
  const size_t need = sa_workspace_bytes(SA_CALL_PHASE2, desc, ctx_len, block_len, t, tail_cap);
  if (need > kScratchBytes)
    return fail(SA_EWORKSPACE,
                "this step needs %zu bytes of scratch, more than the %zu bytes of the library's static array "
                "(use sa_phase2_step with a workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  if ((rc = scratch_address(&ws))) return rc;
  return run_step(desc, q, k_new, v_new, t, k_cache, v_cache, ctx_len, block_len, k_tail, v_tail, tail_cap, tail_len,
                  out, lse, ws, static_cast<hipStream_t>(stream));
}

namespace {

// Chunking of a batched decode step: one chunk length for every sequence, so
// that all their context keys fill one round of resident decode workgroups (two
// where the single-sequence planner measured two faster), after a workgroup
// per sequence and KV head for the tails.
struct BatchPlan {
  int64_t chunk_len;
  int32_t n_chunks[sa::kMaxBatch];
  int32_t n_tail_chunks[sa::kMaxBatch];
  size_t out_off[sa::kMaxBatch];   // workspace byte offsets of each sequence's chunk partials
  size_t lse_off[sa::kMaxBatch];
  size_t bytes;                    // workspace bytes in all
};

BatchPlan batch_plan(const sa_attn_desc* desc, int32_t n_seq, const sa_decode_seq* seqs) {
  BatchPlan p{};
  const int64_t hkv = desc->n_kv_heads, d = desc->head_dim, g = desc->n_q_heads / desc->n_kv_heads;
  int64_t keys = 0;
  for (int i = 0; i < n_seq; ++i) keys += seqs[i].ctx_len * hkv;
  int64_t slots = sa::decode_resident_workgroups(desc->head_dim, g);
  if (slots <= 0) slots = 1024;
  const int64_t tails = (int64_t)n_seq * hkv;
  int64_t w = slots - tails > hkv ? slots - tails : hkv;
  int64_t cl = (keys + w - 1) / w;
  if (g <= 4 && cl * 2 * d * 2 >= (512 << 10) && cl * 2 * d * 2 < (4 << 20)) {
    w = 2 * slots - tails;
    cl = (keys + w - 1) / w;
  }
  cl = (cl + 31) / 32 * 32;
  cl = cl < 128 ? 128 : (cl > 16384 ? 16384 : cl);
  p.chunk_len = cl;
  size_t off = 0;
  for (int i = 0; i < n_seq; ++i) {
    const sa_decode_seq& q = seqs[i];
    const int64_t part_len = q.block_len > q.tail_cap ? q.block_len : q.tail_cap;
    p.n_chunks[i] = (int32_t)((part_len + cl - 1) / cl);
    const int64_t rows_after = q.tail_len + 1;
    const int64_t tc = (rows_after + cl - 1) / cl;
    p.n_tail_chunks[i] = (int32_t)(tc < 1 ? 1 : tc);
    const size_t items = (size_t)(q.ctx_len / q.block_len + 1) * p.n_chunks[i] * desc->n_q_heads;
    p.out_off[i] = off;
    off += (items * d * sizeof(float) + 255) / 256 * 256;
    p.lse_off[i] = off;
    off += (items * sizeof(float) + 255) / 256 * 256;
  }
  p.bytes = off;
  return p;
}

int check_batch(const sa_attn_desc* desc, int32_t n_seq, const sa_decode_seq* seqs) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (desc->dtype != SA_BF16) return fail(SA_ENOTSUP, "batched decode steps are implemented for bf16 only");
  if (desc->n_q_heads / desc->n_kv_heads > 8)
    return fail(SA_ENOTSUP, "batched decode steps take at most 8 query heads per KV head");
  if (n_seq < 1 || n_seq > SA_MAX_BATCH) return fail(SA_EINVAL, "n_seq (%d) must be in [1, %d]", n_seq, SA_MAX_BATCH);
  if (!seqs) return fail(SA_EINVAL, "seqs is NULL");
  for (int i = 0; i < n_seq; ++i) {
    const sa_decode_seq& q = seqs[i];
    if ((rc = check_blocks(q.ctx_len, q.block_len))) return fail(rc, "sequence %d: %s", i, sa_last_error());
    if (q.tail_len < 0 || q.tail_cap > kMaxRows || q.tail_len >= q.tail_cap)
      return fail(SA_EINVAL, "sequence %d: tail_len (%lld) + 1 must fit tail_cap (%lld <= 2^30)", i,
                  (long long)q.tail_len, (long long)q.tail_cap);
    const void* ptrs[8] = {q.q, q.k_new, q.v_new, q.k_cache, q.v_cache, q.k_tail, q.v_tail, q.out};
    if ((rc = check_ptrs("q, k_new, v_new, k_cache, v_cache, k_tail, v_tail, out", 8, ptrs)))
      return fail(rc, "sequence %d: %s", i, sa_last_error());
    if (q.lse && !aligned16(q.lse)) return fail(SA_EINVAL, "sequence %d: lse is not 16-byte aligned", i);
  }
  return SA_OK;
}

}  // namespace

size_t sa_decode_batch_workspace_bytes(const sa_attn_desc* desc, int32_t n_seq, const sa_decode_seq* seqs) {
  if (check_batch(desc, n_seq, seqs) != SA_OK) return 0;
  return batch_plan(desc, n_seq, seqs).bytes;
}

int sa_decode_step_batched(const sa_attn_desc* desc, int32_t n_seq, const sa_decode_seq* seqs, void* workspace,
                           size_t workspace_bytes, void* stream) {
  int rc = check_batch(desc, n_seq, seqs);
  if (rc) return rc;
  const BatchPlan plan = batch_plan(desc, n_seq, seqs);
  if (workspace_bytes < plan.bytes || !workspace)
    return fail(SA_EWORKSPACE, "workspace of %zu bytes given, %zu needed", workspace_bytes, plan.bytes);
  if (!aligned16(workspace)) return fail(SA_EINVAL, "workspace is not 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const sa::RopeTable rt = rope_table(desc);
  char* ws = static_cast<char*>(workspace);
  const int32_t hq = desc->n_q_heads, hkv = desc->n_kv_heads, d = desc->head_dim;

  sa::Phase2Batch pb{};
  sa::MergeBatch mb{};
  pb.n_seq = mb.n_seq = n_seq;
  for (int i = 0; i < n_seq; ++i) {
    const sa_decode_seq& q = seqs[i];
    const int64_t pos = q.ctx_len + q.tail_len;
    float* ws_out = reinterpret_cast<float*>(ws + plan.out_off[i]);
    float* ws_lse = reinterpret_cast<float*>(ws + plan.lse_off[i]);
    const int32_t n_ctx = (int32_t)(q.ctx_len / q.block_len);
    pb.seq[i] = sa::Phase2Args{q.q, q.k_cache, q.v_cache, q.k_tail, q.v_tail, ws_out, ws_lse, 1, pos, q.ctx_len,
                               q.block_len, q.tail_cap, q.tail_len + 1, q.ctx_len, plan.chunk_len, n_ctx,
                               plan.n_chunks[i], hq, hkv, desc->softmax_scale * kLog2eF, plan.n_tail_chunks[i],
                               q.k_new, q.v_new, 1};   // the decode kernel appends the new row itself
    pb.begin[i + 1] = pb.begin[i] + (int64_t)hkv * (plan.n_tail_chunks[i] + (int64_t)n_ctx * plan.n_chunks[i]);
    // the tail's chunk slots past its workgroups hold lse = -inf: left out of the merge
    mb.seq[i] = sa::MergeArgs{ws_out, ws_lse, q.out, q.lse, (int64_t)n_ctx * plan.n_chunks[i] + plan.n_tail_chunks[i],
                              hq, 1, d};
    mb.begin[i + 1] = mb.begin[i] + hq;
  }
  hipError_t e = sa::launch_phase2_decode_batch(pb, rt, d, hq / hkv, s);
  if (e != hipSuccess) return hip_status(e, "batched decode kernel");
  return hip_status(sa::launch_merge_wide_batch(mb, true, s), "batched merge kernel");
}

int sa_phase2_merge(int32_t n_parts, int64_t t_q, int32_t n_q_heads, int32_t head_dim, const float* out_part,
                    const float* lse_part, void* out, int32_t out_dtype, float* lse, void* stream) {
  if (n_parts < 1 || t_q < 1 || n_q_heads < 1) return fail(SA_EINVAL, "n_parts, t_q, n_q_heads must be >= 1");
  if (head_dim != 64 && head_dim != 128) return fail(SA_ENOTSUP, "head_dim %d not supported", head_dim);
  if (out_dtype != SA_F32 && out_dtype != SA_BF16) return fail(SA_EINVAL, "unknown out_dtype %d", out_dtype);
  const void* ptrs[3] = {out_part, lse_part, out};
  int rc = check_ptrs("out_part, lse_part, out", 3, ptrs);
  if (rc) return rc;
  if (lse && !aligned16(lse)) return fail(SA_EINVAL, "lse is not 16-byte aligned");
  if (t_q > kMaxRows || mul_sat(mul_sat(t_q, n_q_heads), 512) > kMaxLaunchThreads)
    return fail(SA_EINVAL, "problem too large for one launch (t_q %lld x %d query heads)", (long long)t_q, n_q_heads);
  sa::MergeArgs ma{out_part, lse_part, out, lse, n_parts, t_q * n_q_heads, 1, head_dim};
  return hip_status(sa::launch_merge(ma, out_dtype == SA_BF16, static_cast<hipStream_t>(stream)),
                    "merge kernel");
}

int sa_calibrate_stream_read(const void* buf, size_t bytes, void* sink, void* stream) {
  if (!buf || !sink || !aligned16(buf) || bytes == 0 || bytes % 16 != 0)
    return fail(SA_EINVAL, "buf/sink must be non-null and 16-byte aligned, bytes a positive multiple of 16");
  return hip_status(sa::launch_stream_read(buf, (int64_t)bytes, static_cast<unsigned*>(sink),
                                           static_cast<hipStream_t>(stream)),
                    "stream-read kernel");
}

int sa_calibrate_mfma(int32_t iters, int32_t n_workgroups, void* sink, void* stream) {
  if (!sink || iters < 1 || n_workgroups < 1) return fail(SA_EINVAL, "sink non-null, iters and n_workgroups >= 1");
  return hip_status(sa::launch_mfma_rate(iters, n_workgroups, static_cast<float*>(sink),
                                         static_cast<hipStream_t>(stream)),
                    "mfma-rate kernel");
}

int sa_device_info(int32_t* n_cus, int32_t* clock_khz, int32_t* mem_clock_khz, int32_t* mem_bus_bits) {
  if (!n_cus || !clock_khz || !mem_clock_khz || !mem_bus_bits) return fail(SA_EINVAL, "null output pointer");
  int dev = 0, v[4] = {0, 0, 0, 0};
  hipError_t e = hipGetDevice(&dev);
  const hipDeviceAttribute_t attr[4] = {hipDeviceAttributeMultiprocessorCount, hipDeviceAttributeClockRate,
                                        hipDeviceAttributeMemoryClockRate, hipDeviceAttributeMemoryBusWidth};
  for (int i = 0; i < 4 && e == hipSuccess; ++i) e = hipDeviceGetAttribute(&v[i], attr[i], dev);
  if (e != hipSuccess) return hip_status(e, "device attributes");
  *n_cus = v[0];
  *clock_khz = v[1];
  *mem_clock_khz = v[2];
  *mem_bus_bits = v[3];
  return SA_OK;
}

}  // extern "C"
