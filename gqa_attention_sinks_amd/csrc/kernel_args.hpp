// Argument blocks passed by value to the kernels, and the host-side launcher
// declarations shared by the C-ABI layer (api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

// Batches of 2 to this many requests run their decode work units longest
// request first (ranked on the host when a host copy of kv_len is given, else
// by every workgroup), unless a window of at most kPlanMinWindow keys makes
// every request's work about the same.
constexpr int kPlanMaxBatch = 256;
constexpr int kPlanMinWindow = 2048;

// Query rows over a paged cache, split into chunks of whole pages; see
// sinkattn_decode_paged and sinkattn_decode_paged_multi in include/sinkattn.h.
struct DecodeArgs {
  const uint16_t* q;          // [rows, Hq, 64] bf16
  const uint16_t* k_pool;     // [num_pages, Hkv, 16, 64] bf16
  const uint16_t* v_pool;
  const int32_t* page_indptr; // [B+1]
  const int32_t* page_indices;
  const int32_t* kv_len;      // [B]
  const int32_t* qo_indptr;   // optional: mixed batch; only requests with one query row are
                              // handled and their row is qo_indptr[b]
  const float* sinks;         // [Hq] or null
  uint16_t* out;              // num_splits == 1: [rows, Hq, 64] bf16
  float* lse;                 // num_splits == 1: optional [rows, Hq]
  float* o_part;              // num_splits > 1: [rows, Hq, S, 64] (rows: B, or total_q with max_rows)
  float* lse_part;            // num_splits > 1: [rows, Hq, S]
  float scale_log2;           // sm_scale * log2(e)
  int32_t batch, num_qo_heads, num_kv_heads, group, num_splits, window;
  int32_t max_rows;           // 0: one query row per request (above); > 0: request b owns
                              // rows qo_indptr[b] .. + min(n_b, max_rows) - 1, partials and
                              // outputs indexed by row
  const uint8_t* custom_mask; // optional with max_rows: bit t * n_k + j of request b's bytes
  const int32_t* mask_indptr; // (from mask_indptr[b]) = row t sees key j
  int32_t planned;            // 1: order[] holds the requests longest first (built on the host)
  uint16_t order[kPlanMaxBatch];
};

struct MergeArgs {
  const float* o_part;        // [rows, H, S, 64]
  const float* lse_part;      // [rows, H, S]
  uint16_t* out;              // [rows, H, 64]
  float* lse;                 // optional [rows, H]
  int32_t rows, num_heads, num_splits;
};

// Causal / sliding-window prefill: a workgroup takes one tile of query rows
// of one query head, or of four heads of one group when the group size is a
// multiple of four.
// Prefill tile order: when a launch has at most kPrefillRankMaxTiles tiles,
// its requests differ in shape and the window is unbounded or longer than
// kPlanMinWindow keys, the tiles run in order of decreasing key count (ties
// request by request); otherwise request by request, each request's longest
// tile first.  A launch of at most kPrefillPlanMax tiles takes that order
// from a plan built on the host (when the caller gives its host copies), and
// its workgroups skip the scan that finds their tile; the plan travels as a
// second kernel argument of its own kernel, so the other launches keep a
// small argument block.
constexpr int kPrefillRankMaxTiles = 256;
constexpr int kPrefillPlanMax = 512;
constexpr int kPrefillTileKeys = 64;        // keys per staged tile

struct PrefillArgs {
  const uint16_t* q;          // [total_q, Hq, 64]
  const int32_t* qo_indptr;   // [B+1]
  const uint16_t* k;          // contiguous [total_kv, Hkv, 64] or pool [P, Hkv, 16, 64]
  const uint16_t* v;
  const int32_t* kv_indptr;   // contiguous: row offsets; paged: offsets into page_indices
  const int32_t* page_indices;
  const int32_t* kv_len;      // paged only
  const float* sinks;
  uint16_t* out;              // [total_q, Hq, 64]
  float* lse;                 // optional [total_q, Hq]
  float scale_log2;
  int32_t batch, num_qo_heads, num_kv_heads, group, window;
  int32_t paged;
  int32_t skip_single_rows;   // requests with one query row are left to the decode kernel
  int32_t num_slots;          // tile slots launched (upper bound on tiles)
};

// The host plan of a prefill launch: slot[s] = request << 16 | tile.
struct PrefillPlan {
  uint32_t slot[kPrefillPlanMax];
};

// Balanced split decode: the batch's live pages cut into equal segments; see
// sinkattn_decode_paged_balanced in include/sinkattn.h.
constexpr int kBalancedMaxBatch = 256;     // the plan of a launch is built in LDS
constexpr int kBalancedWavesPerSimd = 6;   // 4-wave workgroups: six per CU at a time
struct BalancedArgs {
  const uint16_t* q;          // [B, Hq, 64] bf16
  const uint16_t* k_pool;     // [num_pages, Hkv, 16, 64] bf16
  const uint16_t* v_pool;
  const int32_t* page_indptr; // [B+1]
  const int32_t* page_indices;
  const int32_t* kv_len;      // [B]
  const float* sinks;         // [Hq] or null
  uint16_t* out;              // [B, Hq, 64] bf16
  float* lse;                 // optional [B, Hq]
  int32_t* ws_plan;           // workspace: [B+1] live-page prefix (written by workgroup 0)
  int32_t* ws_seg;            // workspace: [B][2] first and last segment of each request (-1: no key)
  float* ws_lse;              // workspace: [slots, Hq] partial LSE (natural log), slot = segment + request
  float* ws_o;                // workspace: [slots, Hq, 64] partial outputs
  float scale_log2;
  int32_t batch, num_qo_heads, num_kv_heads, group, window, num_segments;
};

// Paged KV append with rotary embedding of the new queries and keys; see
// sinkattn_append_paged_kv_rope in include/sinkattn.h.
struct AppendArgs {
  const uint16_t* q;          // optional [T, Hq, 64] bf16 (null: keys only)
  const uint16_t* k_new;      // [T, Hkv, 64] bf16
  const uint16_t* v_new;      // [T, Hkv, 64] bf16
  const int32_t* append_indptr;  // [B+1]
  const int32_t* kv_len;      // [B], counting the appended tokens
  const int32_t* page_indptr; // [B+1]
  const int32_t* page_indices;
  const float* cos_sin;       // [max_pos, 64]: cos of pair f in column f, sin in 32 + f
  uint16_t* q_out;            // [T, Hq, 64] bf16 (may be q)
  uint16_t* k_pool;           // [num_pages, Hkv, 16, 64]
  uint16_t* v_pool;
  int32_t batch, total_new, num_qo_heads, num_kv_heads, max_pos, interleaved;
};

// MoE routing weights; see sinkattn_moe_topk_softmax in include/sinkattn.h.
struct MoeArgs {
  const uint16_t* logits;     // [T, E] bf16
  int32_t* topk_idx;          // [T, K]
  uint16_t* topk_w;           // [T, K] bf16
  int32_t num_tokens, num_experts, top_k;
};

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_verify(const DecodeArgs& a, hipStream_t stream);   // several rows per request
hipError_t launch_decode_balanced(const BalancedArgs& a, hipStream_t stream);   // pieces
hipError_t launch_merge_balanced(const BalancedArgs& a, hipStream_t stream);
hipError_t launch_moe_topk_softmax(const MoeArgs& a, hipStream_t stream);
hipError_t launch_append_rope(const AppendArgs& a, hipStream_t stream);
hipError_t launch_merge(const MergeArgs& a, hipStream_t stream);
// plan: null, or the (request, tile) of each of the a.num_slots tile slots.
hipError_t launch_prefill(const PrefillArgs& a, const PrefillPlan* plan, hipStream_t stream);

}  // namespace sinkattn
