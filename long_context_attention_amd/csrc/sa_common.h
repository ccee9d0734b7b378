// Shared device helpers and the internal launch interface of libstarattn.
// Everything here is gfx950 (CDNA4) code; there is no other target.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16_t;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace sa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kMaxHalfDim = 64;   // head_dim <= 128

// Rotary inverse frequencies theta^(-2j/d), j < d/2, computed on the host in float64.
struct RopeTable {
  double inv_freq[kMaxHalfDim];
};

// cos/sin of pos * inv_freq. The angle is formed and reduced to [-pi, pi] in
// float64 (positions reach 2^20, where a float32 angle would be off by ~0.1 rad);
// only the reduced angle goes through float32 sincos.
__device__ __forceinline__ void rope_cos_sin(int64_t pos, double inv_freq, float* c, float* s) {
  const double a = (double)pos * inv_freq;
  const double r = fma(-rint(a * 0.15915494309189533577), 6.28318530717958647693, a);
  sincosf((float)r, s, c);
}

// The same with the hardware sine and cosine, for values rounded to bf16 next:
// the angle is reduced to [-1/2, 1/2] revolutions in float64 and the hardware
// instructions (which take revolutions) evaluate it, a few instructions
// instead of a library sincosf of about a hundred; their error, 1.2e-7 at most
// on that range against float64 (measured on MI355X), is far below bf16's 2^-9.
__device__ __forceinline__ void rope_cos_sin_hw(int64_t pos, double inv_freq, float* c, float* s) {
  const double rev = (double)pos * inv_freq * 0.15915494309189533577;
  const float r = (float)(rev - rint(rev));
  *s = __builtin_amdgcn_sinf(r);
  *c = __builtin_amdgcn_cosf(r);
}

// The 8 frequencies of rotation-pair group grp, read as four 16-byte loads
// issued together (one wait for all, not one per pair).
__device__ __forceinline__ void rope_freqs8(const double* inv_freq, int grp, double (&f)[8]) {
  typedef double d2 __attribute__((ext_vector_type(2)));
  const d2* src = reinterpret_cast<const d2*>(inv_freq + grp * 8);
  d2 v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = src[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = v[i][0];
    f[2 * i + 1] = v[i][1];
  }
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return (bf16_t)x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Launch parameters (plain structs, passed by value).
// ---------------------------------------------------------------------------
struct RopeStoreArgs {
  const void* k_src;        // [n_rows][n_heads][d]
  const void* v_src;
  void* k_dst;              // [n_heads][dst_rows][d], rows [row0, row0 + n_rows) written
  void* v_dst;
  int64_t n_rows;
  int64_t dst_rows;
  int64_t row0;
  int64_t pos0;
  int32_t n_heads;
  int32_t head_dim;
  // Optional (bf16): the queries of the same rows, [n_rows][q_heads][d]
  // pre-RoPE, rotated at the same positions, scaled by q_scale and stored as
  // bf16 [n_rows][q_heads][d] into q_dst (the attention tile kernel's operand).
  const void* q_src;
  void* q_dst;
  int32_t q_heads;
  float q_scale;
};

struct Phase1Args {
  const void* q;            // [L][Hq][d]
  const void* k_cache;      // [Hkv][L][d]
  const void* v_cache;
  void* out;                // [L][Hq][d]
  int64_t ctx_len;
  int64_t block_len;
  int64_t anchor_len;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  float qk_scale_log2;      // softmax_scale * log2(e)
  int32_t anchor_prev;      // 0: block i > 1 sees the first A rows of block 1; 1: of block i - 1
  // Null, or the anchor's keys rotated at other position IDs for every block
  // i > 1: [Hkv][n - 1][A][d], entry i - 2 for block i (the anchor's values
  // still come from the cache).
  const void* k_anchor;
};

// The anchor's keys (rows [0, A) of the pre-RoPE context keys) rotated at the
// position IDs of up to kAnchorPosBatch blocks per launch, into the per-block
// layout of Phase1Args::k_anchor.
constexpr int kAnchorPosBatch = 64;
struct AnchorKeysArgs {
  const void* k_src;        // [>= A][n_heads][d]
  void* k_dst;              // [n_heads][n_anchors][A][d]
  int64_t anchor_len;
  int64_t n_anchors;        // n - 1
  int64_t first;            // anchor index of pos[0]
  int64_t pos[kAnchorPosBatch];   // first position ID of each anchor in this launch
  int32_t count;            // anchors in this launch
  int32_t n_heads;
  int32_t head_dim;
};

struct Phase2Args {
  const void* q;            // [T][Hq][d]
  const void* k_cache;      // [Hkv][ctx_len][d]
  const void* v_cache;
  const void* k_tail;       // [Hkv][tail_cap][d]
  const void* v_tail;
  float* ws_out;            // [n_parts][n_chunks][T][Hq][d]
  float* ws_lse;            // [n_parts][n_chunks][T][Hq]
  int64_t t_q;
  int64_t q_pos0;
  int64_t ctx_len;
  int64_t block_len;
  int64_t tail_cap;
  int64_t tail_len;
  int64_t tail_pos0;
  int64_t chunk_len;
  int32_t n_ctx_parts;      // n; partition n is the tail
  int32_t n_chunks;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  float qk_scale_log2;
  int32_t n_tail_chunks;    // chunks launched for the tail (decode kernel); <= n_chunks
  // Decode kernel only: when n_new > 0 the last n_new tail rows are the new
  // tokens, whose pre-RoPE K and V ([n_new][Hkv][d]) the kernel rotates and
  // writes into the tail itself (an append fused into the step).
  const void* k_new;
  const void* v_new;
  int32_t n_new;
  // Tile kernel only: null, or the queries already rotated and scaled by
  // qk_scale_log2, bf16 [T][Hq][d] (then the kernel does no RoPE of its own).
  const void* q_rot;
};

// n-way LSE merge over axis 1 of [batch][n][rows][d] (and [batch][n][rows]).
struct MergeArgs {
  const float* o_in;
  const float* lse_in;
  void* o_out;              // [batch][rows][d] in out dtype
  float* lse_out;           // [batch][rows] or null
  int64_t n;
  int64_t rows;
  int64_t batch;
  int32_t head_dim;
};

// Batched decode steps: up to kMaxBatch sequences per launch, their arguments
// passed by value (no device tables, nothing allocated). Work item w of a
// batched launch belongs to the sequence s with begin[s] <= w < begin[s + 1].
constexpr int kMaxBatch = 16;
struct Phase2Batch {
  Phase2Args seq[kMaxBatch];
  int64_t begin[kMaxBatch + 1];   // decode-kernel workgroups
  int32_t n_seq;
};
struct MergeBatch {
  MergeArgs seq[kMaxBatch];
  int64_t begin[kMaxBatch + 1];   // merged rows
  int32_t n_seq;
};

// Kernel choice and chunking of Phase-2 partitions (shared by the workspace
// query and the launch, so both always agree).
enum P2Kernel { P2_VALU = 0, P2_DECODE = 1, P2_TILE = 2 };
struct P2Plan {
  int64_t chunk_len;
  int32_t n_chunks;
  int32_t n_parts;
  int32_t kernel;
};
P2Plan phase2_plan(int64_t ctx_len, int64_t block_len, int64_t t_q, int64_t tail_cap,
                   int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, bool bf16);
struct P2Layout {
  size_t lse_off;    // byte offset of the chunk LSEs
  size_t qrot_off;   // byte offset of the rotated queries (tile kernel)
  size_t bytes;      // workspace bytes in all
};
P2Layout phase2_ws_layout(const P2Plan& p, int64_t t_q, int32_t n_q_heads, int32_t head_dim);

// Launchers: return hipSuccess or the launch error.
hipError_t launch_rope_store(const RopeStoreArgs& a, const RopeTable& rt, bool bf16, hipStream_t s);
hipError_t launch_anchor_keys(const AnchorKeysArgs& a, const RopeTable& rt, bool bf16, hipStream_t s);
hipError_t launch_phase1_valu(const Phase1Args& a, const RopeTable& rt, int head_dim, bool bf16, hipStream_t s);
// `queues`: null (static job order) or kPhase1QueueBytes of device memory for
// the run-time job order (reset by the launch itself).
constexpr size_t kPhase1QueueBytes = 256;
hipError_t launch_phase1_mfma(const Phase1Args& a, const RopeTable& rt, int head_dim, void* queues, hipStream_t s);
hipError_t launch_phase2_decode(const Phase2Args& a, const RopeTable& rt, int head_dim, hipStream_t s);
// Workgroups of the decode kernel that are resident at once on the current
// device (occupancy x compute units), 0 if the runtime cannot tell.
int64_t decode_resident_workgroups(int head_dim, int64_t rows_per_kv);
// *tail_items: how many of the tail partition's chunk slots may hold keys (the
// others get lse = -inf), so a merge may stop before them.
hipError_t launch_phase2_query(const Phase2Args& a, const RopeTable& rt, int head_dim, hipStream_t s,
                               int32_t* tail_items);
hipError_t launch_phase2_valu(const Phase2Args& a, const RopeTable& rt, int head_dim, bool bf16, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, bool out_bf16, hipStream_t s);
// Batched forms (bf16 decode steps of several sequences, one launch each).
hipError_t launch_phase2_decode_batch(const Phase2Batch& b, const RopeTable& rt, int head_dim, int rows_per_kv,
                                      hipStream_t s);
hipError_t launch_merge_wide_batch(const MergeBatch& b, bool out_bf16, hipStream_t s);
hipError_t launch_stream_read(const void* buf, int64_t bytes, unsigned* sink, hipStream_t s);
hipError_t launch_mfma_rate(int iters, int n_workgroups, float* sink, hipStream_t s);

}  // namespace sa
