/*
 * sinkattn.h -- C ABI of libsinkattn: grouped-query flash attention with
 * per-head learned attention sinks on AMD MI355X (gfx950).
 *
 * What is computed.  Perplexity blog "GPT-OSS on day 0" (French rendering
 * "GPT-OSS au jour J"), sections "GPT-OSS on Hopper" (GQA with one pretrained
 * sink per head, counted in the softmax) and "Kernels for GPT-OSS > Sink
 * attention" (the sink is an extra term of the softmax next to the Q.K
 * products; the streaming softmax keeps a running max m and a scale d, which
 * start at the head's sink value and 1; when the KV sequence is split into
 * blocks only the first block carries the sink).  For request b with n_q query
 * rows and n_k cached keys, query row t, query head h, KV head g = h / (Hq/Hkv):
 *
 *   p    = n_k - n_q + t                      (bottom-right causal position)
 *   keys = { j : lo <= j <= p },  lo = max(0, p - window + 1) if window > 0 else 0
 *   Z    = exp(sink[h]) + sum_j exp(sm_scale * <q[t,h], k[j,g]>)
 *   out  = sum_j exp(sm_scale * <q[t,h], k[j,g]>) / Z * v[j,g]
 *   lse  = ln Z                              (natural log; includes the sink)
 *
 * The sink is on the scaled-logit scale (sm_scale never multiplies it) and
 * has no value row.  A NULL sinks pointer means every sink is -inf, which is
 * plain softmax attention.
 *
 * KV metadata.  "Accelerating Sonar through speculation" (Perplexity blog,
 * Greek rendering), section "Inference with speculative decoding": the
 * scheduler allocates KV-cache pages per request and the CPU builds the
 * metadata (index pointers, page tables) that configures the attention
 * kernel, then copies it to GPU memory.  Here that metadata is the
 * sinkattn_kv descriptor below.
 *
 * Conventions for every entry point:
 *  - Pointers are device memory unless documented "host".  bf16 tensors are
 *    raw 16-bit patterns.  All tensors are dense, row-major, contiguous.
 *  - Layouts: q and out [total_q, Hq, 64]; contiguous K/V [total_kv, Hkv, 64];
 *    paged K/V pools [num_pages, Hkv, 16, 64] (one (page, KV head) block is
 *    2 KiB contiguous); sinks [Hq] fp32; lse [total_q, Hq] fp32.
 *  - Ownership: the caller allocates and owns every buffer.  The library
 *    allocates no device memory, never synchronises the host, and keeps no
 *    device state between calls; work is enqueued on `stream` (a hipStream_t,
 *    NULL = the default stream) and is safe to capture in a HIP graph.
 *  - Errors: argument problems are found on the host before anything is
 *    enqueued, so a non-OK status means nothing was launched and nothing was
 *    written.  SINKATTN_ERR_HIP reports a failed launch.  Device-resident
 *    metadata (kv_len, page ids, index pointers) is trusted by the attention
 *    calls: checking it there would need a host synchronisation.  A caller
 *    that builds the metadata on the CPU (the usual case) checks its host
 *    copy with sinkattn_validate_kv_host before copying it to the GPU.
 *  - Thread safety: entry points may be called concurrently from several
 *    host threads; sinkattn_last_error() is per thread.
 *  - Supported shapes: head_dim 64, page_size 16, 1 <= Hq/Hkv <= 16,
 *    Hq % Hkv == 0.
 *  - Value range (precondition of sinkattn_prefill, sinkattn_decode_paged
 *    and sinkattn_decode_paged_multi): the P.V products run on fp16 matrix
 *    instructions (fp16 weights carry three more significand bits than
 *    bf16), so V is converted from bf16 to fp16 when it is staged.  Every V
 *    value of every key a request holds (logical keys 0 .. n_k - 1, also
 *    those a mask or window hides: whole pages and tiles are staged) must
 *    satisfy |v| <= 65280, the largest bf16 magnitude below fp16's overflow
 *    at 65520.  All such values convert exactly, except magnitudes below
 *    2^-14, which become fp16 subnormals (absolute change below 2^-24).  A
 *    larger |v| is not detected: the output of the affected rows is
 *    undefined (inf or NaN).  Q and K have no such limit (their products run
 *    in bf16), and neither do the sinks.
 */
#ifndef SINKATTN_H_
#define SINKATTN_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SINKATTN_ABI_VERSION 8
#define SINKATTN_HEAD_DIM 64
#define SINKATTN_PAGE_SIZE 16
#define SINKATTN_MAX_SPLITS 256
#define SINKATTN_MAX_DECODE_ROWS 8
#define SINKATTN_MAX_EXPERTS 512
#define SINKATTN_MAX_TOP_K 8
#define SINKATTN_MAX_BALANCED_BATCH 256
#define SINKATTN_NOALLOC_SCRATCH_BYTES (8u << 20) /* partials of sinkattn_decode_paged_noalloc */

typedef enum {
  SINKATTN_OK = 0,
  SINKATTN_ERR_INVALID_ARG = 1, /* NULL required pointer, Hq % Hkv != 0, batch < 1, bad split
                                   count, window < 0, sm_scale not finite or <= 0 ... */
  SINKATTN_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement: head_dim
                                   != 64, page_size != 16, Hq/Hkv > 16 */
  SINKATTN_ERR_HIP = 3          /* a kernel launch failed; sinkattn_last_error() has the text */
} sinkattn_status;

/* Where the keys and values of the batch live (a host struct holding device
 * pointers).
 *   paged == 0:  k, v are [total_kv, Hkv, 64] bf16; request b owns rows
 *                kv_indptr[b] .. kv_indptr[b+1]-1, so n_k = kv_indptr[b+1] -
 *                kv_indptr[b]; kv_len and page_indices are ignored.
 *   paged == 1:  k, v are pools [num_pages, Hkv, 16, 64] bf16; request b's
 *                logical key j lives in slot j % 16 of physical page
 *                page_indices[kv_indptr[b] + j / 16]; n_k = kv_len[b].
 *                Slots past a request's last key are never read.
 *   kv_indptr [B+1] int32 and kv_len [B] int32 are device arrays; page ids are
 *   int32 but byte offsets into the pools are computed in 64 bits.
 *   num_pages: the capacity of k and v -- paged: pages in each pool;
 *   contiguous: rows of k and v.  The attention calls do not read it (the
 *   metadata is device memory); sinkattn_validate_kv_host checks a host copy
 *   of the metadata against it. */
typedef struct sinkattn_kv {
  const void* k;
  const void* v;
  int32_t paged;
  int32_t page_size;             /* paged: must be 16 */
  const int32_t* kv_indptr;
  const int32_t* page_indices;   /* paged only */
  const int32_t* kv_len;         /* paged only */
  int64_t num_pages;             /* capacity of k and v (pages, or rows when contiguous) */
  /* Optional host copy of kv_len [batch] (NULL: none).  Paged decode calls
   * (sinkattn_decode_paged, _noalloc, _multi, and the decode rows of
   * sinkattn_prefill) run their (request, KV head, chunk) work units longest
   * request first; with this copy the library orders them on the host and
   * passes the order with the launch, instead of every workgroup ranking the
   * batch's lengths ("Accelerating Sonar through speculation", section
   * "Inference with speculative decoding": the host side of the runtime fills
   * the buffers that configure and schedule the attention kernel for each
   * batch).  The tile table of a paged sinkattn_prefill call also takes its
   * order from it (see qo_indptr_host there).  It only orders the work: the
   * results are the same whatever it holds (the lengths the kernels use are
   * always the device kv_len's).  sinkattn_decode_paged_balanced plans its
   * segments on the device and does not read it. */
  const int32_t* kv_len_host;
} sinkattn_kv;

/* Causal or sliding-window prefill over a batch of requests, each with
 * n_q >= 1 new query rows whose own keys are already in the cache (n_q <=
 * n_k).  Chunked prefill and decode rows may be mixed in one call: rows of
 * requests with n_q == 1 are handled by the decode kernel (two launches on
 * `stream`).
 *   q          [total_q, Hq, 64] bf16, request b's rows qo_indptr[b] .. qo_indptr[b+1]-1
 *   qo_indptr  [batch+1] int32 (device)
 *   kv         host pointer to the KV descriptor
 *   sinks      [Hq] fp32 or NULL (no sink)
 *   out        [total_q, Hq, 64] bf16, written
 *   lse        [total_q, Hq] fp32 natural-log LSE (sink included), or NULL
 *   total_q    number of query rows (= qo_indptr[batch]); bounds the launch
 *   window     0 = full causal, W > 0 = each row sees its last W positions
 *              (its own included)
 *   qo_indptr_host  optional host copy of qo_indptr ([batch+1], host memory,
 *              read during the call only).  The CPU-side plan of the launch
 *              ("Accelerating Sonar through speculation", section "Inference
 *              with speculative decoding": the CPU fills the buffers that
 *              configure and schedule the attention kernel): with it the
 *              prefill grid holds exactly the query tiles of the batch, and
 *              a launch of up to 512 tiles takes each workgroup's (request,
 *              tile) from a table built here instead of a scan over the
 *              batch in every workgroup (for a paged call that the kernel
 *              would order by key count, the table also needs
 *              kv->kv_len_host, which only sets the order); without it the
 *              grid is sized from total_q and batch and the surplus
 *              workgroups exit at once.  It must equal qo_indptr on the
 *              device.  Results are identical either way. */
sinkattn_status sinkattn_prefill(const void* q, const int32_t* qo_indptr, const sinkattn_kv* kv,
                                 const float* sinks, void* out, float* lse, int32_t batch,
                                 int32_t total_q, int32_t num_qo_heads, int32_t num_kv_heads,
                                 int32_t head_dim, float sm_scale, int32_t window,
                                 const int32_t* qo_indptr_host, void* stream);

/* One query token per request over a paged KV cache, split along the KV
 * sequence into num_splits chunks of whole pages: with n_pages =
 * ceil(n_k / 16) and ppc = ceil(n_pages / num_splits), chunk c covers pages
 * [c*ppc, min((c+1)*ppc, n_pages)) (chunks may be empty).  The sink enters
 * chunk 0 only ("Kernels for GPT-OSS > Sink attention").  The query of
 * request b sits at position kv_len[b] - 1.
 *   q          [batch, Hq, 64] bf16
 *   kv         paged descriptor (kv->paged must be 1)
 *   num_splits 1 .. SINKATTN_MAX_SPLITS
 *   out        num_splits == 1: [batch, Hq, 64] bf16 (required).
 *              num_splits > 1: optional; when given, the partials are merged
 *              into it by a second launch (same as calling sinkattn_merge).
 *   o_part     num_splits > 1: [batch, Hq, num_splits, 64] fp32, each chunk
 *              normalised by its own denominator; empty chunks hold 0.
 *   lse_part   num_splits > 1: [batch, Hq, num_splits] fp32 natural-log
 *              partial LSE: -inf for an empty chunk, the sink for an empty
 *              chunk 0.  Both ignored (may be NULL) when num_splits == 1.
 *   lse        optional [batch, Hq] fp32 final LSE (written with out). */
sinkattn_status sinkattn_decode_paged(const void* q, const sinkattn_kv* kv, const float* sinks,
                                      int32_t num_splits, void* out, float* o_part,
                                      float* lse_part, float* lse, int32_t batch,
                                      int32_t num_qo_heads, int32_t num_kv_heads,
                                      int32_t head_dim, float sm_scale, int32_t window,
                                      void* stream);

/* One query token per request over a paged KV cache, the batch's work split
 * into equal segments: the same results as sinkattn_decode_paged (out, lse),
 * computed with a split that does not depend on the mix of request lengths.
 * "GPT-OSS on day 0", section "Kernels for GPT-OSS > Sink attention": the
 * attention is split into blocks along the KV sequence, only the first block
 * of a request carries its sink, and the blocks' partial softmaxes are
 * merged.  The blocks: a request's live pages are those holding the keys its
 * query row sees (keys max(0, n_k - window) .. n_k - 1; all keys when window
 * == 0); the batch's live pages, request after request, form one list of T
 * pages, and segment s (0 <= s < num_segments) holds list positions
 * [floor(s T / N), floor((s + 1) T / N)).  A request's part of a segment is
 * one block.  One workgroup per (segment, KV head) walks its segment; a
 * request that lies in one segment is finished there, the blocks of the
 * others are merged by a second launch.
 *   q            [batch, Hq, 64] bf16; the query of request b sits at position
 *                kv_len[b] - 1
 *   kv           paged descriptor (kv->paged must be 1)
 *   num_segments 1 .. 65536; sinkattn_pick_num_segments gives the count that
 *                fills the GPU once
 *   workspace    device memory of at least
 *                sinkattn_decode_balanced_workspace_bytes(batch, Hq,
 *                num_segments) bytes, 16-byte aligned, owned by the caller;
 *                its contents on entry do not matter.  On return it holds
 *                int32 plan[batch + 1] (the live-page prefix: request b owns
 *                list positions plan[b] .. plan[b+1] - 1) and int32
 *                seg[batch][2] (each request's first and last segment, -1
 *                for a request without keys), then (at the next multiple of
 *                256 bytes) fp32 lse[slots][Hq], then fp32
 *                o[slots][Hq][64], slots = num_segments + batch: the blocks of
 *                the requests that span several segments, request b's block
 *                in segment s at slot s + b, each normalised by its own
 *                denominator with its natural-log LSE (the first block with
 *                the sink).  Calls that share a workspace must not overlap.
 *   out          [batch, Hq, 64] bf16, written; lse optional [batch, Hq] fp32
 * batch <= SINKATTN_MAX_BALANCED_BATCH (the plan of a launch is built in the
 * workgroups' shared memory); larger batches get SINKATTN_ERR_UNSUPPORTED and
 * are served by sinkattn_decode_paged.  A request with no key gets out = 0,
 * lse = sink. */
sinkattn_status sinkattn_decode_paged_balanced(const void* q, const sinkattn_kv* kv, const float* sinks,
                                               int32_t num_segments, void* workspace,
                                               int64_t workspace_bytes, void* out, float* lse,
                                               int32_t batch, int32_t num_qo_heads,
                                               int32_t num_kv_heads, int32_t head_dim, float sm_scale,
                                               int32_t window, void* stream);

/* The two launches of sinkattn_decode_paged_balanced one at a time (same
 * arguments and contract): _pieces walks the segments (requests that lie in
 * one segment get their out and lse; the others leave their blocks in the
 * workspace), then _merge (with the workspace of that call) merges those
 * blocks into out and lse and writes the requests without keys.  For callers
 * that time or schedule the two apart. */
sinkattn_status sinkattn_decode_paged_balanced_pieces(const void* q, const sinkattn_kv* kv, const float* sinks,
                                                      int32_t num_segments, void* workspace,
                                                      int64_t workspace_bytes, void* out, float* lse,
                                                      int32_t batch, int32_t num_qo_heads,
                                                      int32_t num_kv_heads, int32_t head_dim,
                                                      float sm_scale, int32_t window, void* stream);
sinkattn_status sinkattn_merge_balanced(const float* sinks, int32_t num_segments, const void* workspace,
                                        int64_t workspace_bytes, void* out, float* lse, int32_t batch,
                                        int32_t num_qo_heads, int32_t head_dim, void* stream);

/* Host-only: bytes of workspace sinkattn_decode_paged_balanced needs (-1 on
 * invalid arguments). */
int64_t sinkattn_decode_balanced_workspace_bytes(int32_t batch, int32_t num_qo_heads, int32_t num_segments);

/* Host-only: the segment count for sinkattn_decode_paged_balanced that lets
 * every (segment, KV head) workgroup of one launch run at once on the current
 * device (six per compute unit). */
int32_t sinkattn_pick_num_segments(int32_t num_kv_heads);

/* Host-only: the segment rule of sinkattn_decode_paged_balanced, for callers
 * and tests.  kv_len_host [batch] (host); segs_host [batch, 2] (host) receives
 * each request's first and last segment (-1, -1 for a request without keys). */
sinkattn_status sinkattn_balanced_segments(const int32_t* kv_len_host, int32_t batch, int32_t window,
                                           int32_t num_segments, int32_t* segs_host);

/* sinkattn_decode_paged for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same computation, arguments and results as
 * sinkattn_decode_paged with out given (the split partials are merged into
 * out, and lse, if given, gets the final LSE), but the caller passes no
 * partial buffers: for num_splits > 1 they live in a device array owned by
 * the library, SINKATTN_NOALLOC_SCRATCH_BYTES (8 MiB) per GPU, held until
 * the process ends.  Its address on the current device is looked up on the
 * first call there (`stream` must belong to the current device).  The
 * partials need batch * Hq * num_splits * 65 * 4 bytes (plus 256 of
 * alignment); larger calls are rejected with SINKATTN_ERR_INVALID_ARG before
 * anything is enqueued -- use sinkattn_decode_paged with caller-owned
 * partials for them.  No call allocates or frees memory.  Every call on one
 * GPU shares that array: calls that may overlap on a GPU (concurrent streams,
 * several host threads) race and must be ordered by the caller; nothing in it
 * needs clearing between calls (each call writes every partial it reads). */
sinkattn_status sinkattn_decode_paged_noalloc(const void* q, const sinkattn_kv* kv, const float* sinks,
                                              int32_t num_splits, void* out, float* lse, int32_t batch,
                                              int32_t num_qo_heads, int32_t num_kv_heads,
                                              int32_t head_dim, float sm_scale, int32_t window,
                                              void* stream);

/* Several query rows per request over a paged KV cache, split along the KV
 * sequence like sinkattn_decode_paged: the step in which the target model
 * scores a few proposed tokens at once ("Accelerating Sonar through
 * speculation", sections "Speculative decoding" and "Inference with
 * speculative decoding").  Request b owns query rows qo_indptr[b] ..
 * qo_indptr[b+1]-1; its row t sits at position kv_len[b] - n_q + t
 * (bottom-right causal: the proposed tokens' own keys are already in the
 * cache), and a window W > 0 limits each row to its last W positions.  The
 * chunks are the request's pages dealt out as in sinkattn_decode_paged (the
 * same for all of its rows), the sink enters chunk 0 only ("Kernels for
 * GPT-OSS > Sink attention").  One workgroup per (request, KV head, chunk)
 * reads each page once for all G = Hq/Hkv heads and all rows of the request.
 *   q          [total_q, Hq, 64] bf16
 *   qo_indptr  [batch+1] int32 (device); every request must have at most
 *              max_qo_len rows (not checked: the offsets are device memory;
 *              the results of a request with more are undefined); a request
 *              with no row is skipped
 *   custom_mask optional (device, NULL = the causal rule above): a draft
 *              tree verified in one step (tree attention, "Accelerating
 *              Sonar through speculation", section "Speculative decoding":
 *              the target scores the drafted tokens in one pass).  Request b's
 *              mask starts at byte mask_indptr[b]; bit t * kv_len[b] + j of it
 *              (bit i in byte i / 8 at position i % 8) says whether row t
 *              sees key j.  It replaces the causal rule and needs window == 0;
 *              the sink is not a key and is never masked.  A row with no
 *              visible key gets out = 0, lse = sink.
 *   mask_indptr [batch+1] int32 byte offsets (device), required with custom_mask
 *   max_qo_len 1 .. SINKATTN_MAX_DECODE_ROWS, with (Hq/Hkv) * max_qo_len <= 64
 *   kv         paged descriptor (kv->paged must be 1)
 *   num_splits 1 .. SINKATTN_MAX_SPLITS
 *   out        num_splits == 1: [total_q, Hq, 64] bf16 (required).
 *              num_splits > 1: optional; when given, the partials are merged
 *              into it by a second launch (same as sinkattn_merge over
 *              total_q rows).
 *   o_part     num_splits > 1: [total_q, Hq, num_splits, 64] fp32, each chunk
 *              normalised by its own denominator; empty chunks hold 0.
 *   lse_part   num_splits > 1: [total_q, Hq, num_splits] fp32 natural-log
 *              partial LSE: -inf for an empty chunk, the sink for an empty
 *              chunk 0.  Both ignored (may be NULL) when num_splits == 1.
 *   lse        optional [total_q, Hq] fp32 final LSE (written with out).
 * A row whose position is below 0 (n_q > kv_len) sees no key: out = 0,
 * lse = sink. */
sinkattn_status sinkattn_decode_paged_multi(const void* q, const int32_t* qo_indptr,
                                            const uint8_t* custom_mask, const int32_t* mask_indptr,
                                            const sinkattn_kv* kv, const float* sinks,
                                            int32_t num_splits, void* out, float* o_part,
                                            float* lse_part, float* lse, int32_t batch,
                                            int32_t total_q, int32_t max_qo_len,
                                            int32_t num_qo_heads, int32_t num_kv_heads,
                                            int32_t head_dim, float sm_scale, int32_t window,
                                            void* stream);

/* Append new tokens' keys and values to a paged KV cache, with rotary
 * position embedding applied to the new keys and (optionally) the new queries:
 * the step just upstream of attention for a decode or verify batch.  "GPT-OSS
 * on day 0", section "GPT-OSS on Hopper" (the models use YaRN rotary position
 * encoding); "Accelerating Sonar through speculation", section "Inference
 * with speculative decoding" (per-request pages, CPU-built page tables).  The
 * pages give neither YaRN's constants nor the pair layout, so the rotation
 * comes from the caller's table and layout flag:
 *   pair f (0..31) is (x[f], x[f + 32]) (interleaved = 0) or (x[2f], x[2f + 1])
 *   (interleaved = 1); at position p it becomes
 *   (a cos - b sin, b cos + a sin) with cos = cos_sin[p][f], sin = cos_sin[p][32 + f].
 * Request b appends n_b = append_indptr[b+1] - append_indptr[b] tokens, which
 * take positions kv_len[b] - n_b .. kv_len[b] - 1 (kv_len already counts them,
 * as the attention call that follows does); position p lives in page
 * page_indices[kv_indptr[b] + p / 16], slot p % 16.
 *   q        optional [total_new, Hq, 64] bf16 (NULL: keys only)
 *   k_new, v_new [total_new, Hkv, 64] bf16
 *   append_indptr [batch+1] int32 (device)
 *   kv       paged descriptor (kv->paged must be 1); its pools are written at
 *            the new tokens' slots only
 *   cos_sin  [max_pos, 64] fp32 (device, 16-byte aligned)
 *   q_out    [total_new, Hq, 64] bf16, written (may equal q); NULL when q is NULL
 * Results are rounded to bf16 from fp32 arithmetic; values are copied
 * exactly.  A token whose position falls outside [0, max_pos) is not written
 * (its query row either).  Two appends that hit the same slot race.  With
 * total_new == 0 nothing is read or written and k_new, v_new, q and q_out may
 * be NULL. */
sinkattn_status sinkattn_append_paged_kv_rope(const void* q, const void* k_new, const void* v_new,
                                              const int32_t* append_indptr, const sinkattn_kv* kv,
                                              const float* cos_sin, int32_t max_pos,
                                              int32_t interleaved, void* q_out, int32_t batch,
                                              int32_t total_new, int32_t num_qo_heads,
                                              int32_t num_kv_heads, int32_t head_dim,
                                              void* stream);

/* MoE routing weights of GPT-OSS: for every token the top_k largest router
 * logits and the softmax over those top_k logits alone ("GPT-OSS on day 0",
 * sections "GPT-OSS on Hopper" and "Kernels for GPT-OSS > MoE": softmax after
 * the top-K selection, over the selected experts only, with the expert
 * weights computed in bfloat16 precision).  The selection compares the bf16
 * logits exactly; equal logits (-0 equals +0) rank the lower expert index
 * first.  The softmax runs in fp32 on the bf16 logits and is rounded to bf16.
 *   logits    [num_tokens, num_experts] bf16 (device); NaN logits give
 *             unspecified picks
 *   topk_idx  [num_tokens, top_k] int32, written: expert ids, largest logit
 *             first
 *   topk_w    [num_tokens, top_k] bf16, written: the weights, same order
 *   1 <= num_experts <= SINKATTN_MAX_EXPERTS, 1 <= top_k <=
 *   min(SINKATTN_MAX_TOP_K, num_experts).  With num_tokens == 0 nothing is
 *   read or written and the three buffers may be NULL. */
sinkattn_status sinkattn_moe_topk_softmax(const void* logits, int32_t num_tokens, int32_t num_experts,
                                          int32_t top_k, int32_t* topk_idx, void* topk_w, void* stream);

/* Log-sum-exp merge of split partials: "GPT-OSS on day 0", section "Kernels
 * for GPT-OSS > Sink attention" -- attention split into blocks along the KV
 * sequence, the sink carried by the first block only; each block's partial
 * is a softmax over its own keys with its own log-sum-exp, and the blocks
 * combine into the softmax over all keys.  Per (row, head), with
 * M = max_c lse_c and w_c = exp(lse_c - M), out = sum_c w_c o_c / sum_c w_c
 * and lse = M + ln sum_c w_c; all-(-inf) rows give out = 0, lse = -inf.  The
 * sink needs no argument here: it is already inside the first block's
 * partial (its LSE includes it, its output carries no value for it).
 *   o_part [rows, num_heads, num_splits, 64] fp32, lse_part [rows, num_heads,
 *   num_splits] fp32; out [rows, num_heads, 64] bf16; lse_out optional
 *   [rows, num_heads] fp32. */
sinkattn_status sinkattn_merge(const float* o_part, const float* lse_part, int32_t rows,
                               int32_t num_heads, int32_t num_splits, int32_t head_dim, void* out,
                               float* lse_out, void* stream);

/* Host-only: the chunk rule used by sinkattn_decode_paged, for callers and
 * tests.  kv_len_host [batch] (host), bounds_host [batch, num_splits, 2]
 * (host) receives each chunk's token range [lo, hi). */
sinkattn_status sinkattn_split_bounds(const int32_t* kv_len_host, int32_t batch,
                                      int32_t page_size, int32_t num_splits,
                                      int32_t* bounds_host);

/* Host-only: a split count for sinkattn_decode_paged chosen for the shape
 * (kv_len_host [batch], host): enough (request, KV head, chunk) work units to
 * fill the GPU without making chunks shorter than a few pages. */
int32_t sinkattn_pick_num_splits(const int32_t* kv_len_host, int32_t batch, int32_t num_kv_heads);

/* Host-only: a split count for sinkattn_decode_paged_multi (kv_len_host
 * [batch], host; max_qo_len and with_mask as in the call).  That kernel runs
 * two workgroups per compute unit, so it is given fewer, longer chunks than
 * the one-row rule gives: about 4/3 of the workgroups the GPU holds at once
 * (twice that with a mask), chunks of at least 16 pages, at most 16 of them.
 * Returns 1 on invalid arguments. */
int32_t sinkattn_pick_num_splits_multi(const int32_t* kv_len_host, int32_t batch, int32_t num_qo_heads,
                                       int32_t num_kv_heads, int32_t max_qo_len, int32_t with_mask);

/* Host-only: check a host copy of a batch's KV metadata before it is copied to
 * the GPU ("Accelerating Sonar through speculation", section "Inference with
 * speculative decoding": the CPU builds the page metadata that configures
 * the attention kernel and copies it to GPU memory).  kv supplies paged,
 * page_size and num_pages (its device pointers are not read); the three
 * arrays are host memory: kv_indptr_host [batch+1], and when paged
 * page_indices_host [kv_indptr_host[batch]] and kv_len_host [batch].
 * Checks, for every request b:
 *   paged:      0 <= kv_indptr[b] <= kv_indptr[b+1]; kv_len[b] >= 0;
 *               ceil(kv_len[b] / 16) <= kv_indptr[b+1] - kv_indptr[b] (the
 *               pages the attention calls read); each of those page ids in
 *               [0, num_pages); num_pages >= 1
 *   contiguous: 0 <= kv_indptr[b] <= kv_indptr[b+1] <= num_pages
 * Returns SINKATTN_OK, or SINKATTN_ERR_INVALID_ARG with the first offending
 * entry named in sinkattn_last_error().  Page ids past a request's live pages
 * are not read by the kernels and not checked. */
sinkattn_status sinkattn_validate_kv_host(const sinkattn_kv* kv, const int32_t* kv_indptr_host,
                                          const int32_t* page_indices_host,
                                          const int32_t* kv_len_host, int32_t batch);

const char* sinkattn_status_string(sinkattn_status status);
const char* sinkattn_last_error(void); /* message of this thread's last failing call */
const char* sinkattn_last_hip_error(void); /* the same message (name kept for HIP-error callers) */
int32_t sinkattn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SINKATTN_H_ */
