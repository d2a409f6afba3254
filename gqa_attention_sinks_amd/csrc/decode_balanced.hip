// Balanced paged decode with per-head attention sinks: the batch's work split
// into equal segments, and the merge of the pieces that cross segments.
//
// Method: Perplexity blog "GPT-OSS on day 0" (French rendering "GPT-OSS au
// jour J"), section "Kernels for GPT-OSS > Sink attention": attention is split
// into blocks along the KV sequence, the streaming softmax of a block keeps a
// running max m and a scale d, only the first block starts from the head's
// sink, and the blocks' partial softmaxes combine into the whole one.  Paged
// KV and CPU-built page metadata: "Accelerating Sonar through speculation",
// section "Inference with speculative decoding".
//
// The blocks here are not a fixed number per request: the batch's live pages
// (the pages holding keys that a request's query row sees), request after
// request, form one list of T pages, and segment s of N holds list positions
// [floor(s T / N), floor((s + 1) T / N)).  Every segment carries the same
// number of pages (to one), whatever the mix of request lengths, so the
// workgroups of one launch finish together.  A request's part of a segment is
// a piece; its first piece carries the sink.
//
// Work decomposition (gfx950, 64-lane waves):
//   workgroup = (segment s, KV head g), four waves, six waves per SIMD (the
//   library's segment count fills the GPU in one round).  Each workgroup first
//   builds the plan in LDS (every request's live pages and their prefix, at
//   most 256 requests), then walks the requests of its segment.  The waves
//   take a piece's pages round robin (wave w: pages w, w + 4, ...), and at
//   the piece's end merge their softmax states through LDS:
//     * a piece that is a whole request (it starts and ends inside the
//       segment) is final: bf16 output and LSE are written directly;
//     * otherwise the piece's partial (its output normalised by its own
//       denominator, and its natural-log LSE) goes to workspace slot s + r
//       (r the request), and the merge kernel below combines the slots.
//   Per page (16 keys x 64 dims = 2 KiB per KV head, contiguous in the pool):
//     S^T[16 keys x 16 heads] = K . Q^T   -> 2 x MFMA 16x16x32 bf16 (K straight
//       from HBM into the A operand; the G <= 16 query heads of KV head g are
//       the columns; Q^T staged in LDS once per piece)
//     online softmax in base 2 on the accumulator (each lane: one head, 4 keys)
//     O^T[64 dims x 16 heads] += V^T . P^T -> 4 x MFMA 16x16x16 fp16 (V
//       converted to fp16, staged in LDS, read back with ds_read_b64_tr_b16)
//   The fp16 weights are taken relative to the running key maximum and the
//   sink is folded in at the end (fold_sink), which gives exactly the state of
//   the sink-seeded recurrence after the same keys.

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace sinkattn {
namespace {

constexpr int kNW = 4;                                 // waves per workgroup
constexpr int kThreads = kNW * 64;
constexpr int kPageBytes = kPageSize * kHeadDim * 2;   // one (page, KV head) block: 2 KiB
constexpr float kFloatMax = 3.402823466e38f;

static_assert(kBalancedMaxBatch <= kThreads, "one thread per request builds the plan");

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Byte offset of 16-byte chunk `chunk` of row `key` in a [16][64] page staged
// in LDS, XOR-swizzled so the transposed reads spread over all banks.
__device__ __forceinline__ int page_swizzle(int key, int chunk) {
  return key * 128 + ((chunk ^ (key & 7)) << 4);
}

// LDS of a workgroup: the plan tables, then a region that holds the V
// staging pages and the Q^T operands while pages are processed, and the
// four waves' softmax states while a piece is merged.
struct BalancedSmem {
  int pre[kBalancedMaxBatch + 1];   // live-page prefix: request r owns list positions [pre[r], pre[r+1])
  int nk[kBalancedMaxBatch];        // KV length
  int base[kBalancedMaxBatch];      // index in page_indices of the request's first live page
  int wave_sum[kNW];
  union {
    struct {
      uint8_t stage[kNW][kPageBytes];
      u32x4 q[2][64];               // Q^T operands: [k half][lane], lane = (column, 16-dim group)
    } run;
    struct {
      float m[kNW][16];
      float d[kNW][16];
      float o[kNW][16][kHeadDim];
    } merge;
  } u;
};

// A value the compiler must treat as new at this point: lane-derived
// addresses are then recomputed in each piece instead of being held (and
// spilled) across the whole segment.
__device__ __forceinline__ int opaque(int x) {
  __asm__ volatile("" : "+v"(x));
  return x;
}

// Segment holding list position f of T (N segments): the s with
// floor(s T / N) <= f < floor((s + 1) T / N).
__device__ __forceinline__ int segment_of(long long f, long long T, long long N) {
  return (int)(((f + 1) * N - 1) / T);
}

// Largest r in [0, B) with pre[r] <= f (f < pre[B]): the request holding list
// position f.
__device__ __forceinline__ int request_of(const int* pre, int B, int f) {
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= f) lo = mid;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kBalancedWavesPerSimd)))
void decode_balanced_kernel(BalancedArgs a) {
  __shared__ __attribute__((aligned(16))) BalancedSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int B = a.batch, W = a.window, G = a.group;
  const int g = blockIdx.x % a.num_kv_heads;
  const int s = blockIdx.x / a.num_kv_heads;

  // ---- plan: live pages of every request and their prefix (one thread each)
  int n_live = 0;
  if (tid < B) {
    const int n_k = a.kv_len[tid];
    const int lo = W > 0 ? max(0, n_k - W) : 0;
    const int first = lo / kPageSize;
    n_live = n_k > 0 ? (n_k + kPageSize - 1) / kPageSize - first : 0;
    sm.nk[tid] = n_k;
    sm.base[tid] = a.page_indptr[tid] + first;
  }
  int incl = n_live;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) sm.wave_sum[wave] = incl;
  __syncthreads();
  int wave_off = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kNW; ++w) {
    wave_off += w < wave ? sm.wave_sum[w] : 0;
    total += sm.wave_sum[w];
  }
  total = __builtin_amdgcn_readfirstlane(total);   // LDS values are uniform: keep them scalar
  if (tid < B) sm.pre[tid] = wave_off + incl - n_live;
  if (tid == 0) sm.pre[B] = total;
  __syncthreads();
  if (blockIdx.x == 0) {                                  // the plan, for the merge kernel
    if (tid < B) {
      const int p = sm.pre[tid];
      a.ws_plan[tid] = p;
      a.ws_seg[2 * tid] = n_live > 0 ? segment_of(p, total, a.num_segments) : -1;
      a.ws_seg[2 * tid + 1] = n_live > 0 ? segment_of(p + n_live - 1, total, a.num_segments) : -1;
    }
    if (tid == 0) a.ws_plan[B] = total;                     // (B may equal the thread count)
  }

  const int S0 = (int)((long long)s * total / a.num_segments);
  const int S1 = (int)((long long)(s + 1) * total / a.num_segments);
  if (S0 >= S1) return;                                   // uniform: an empty segment
  const int r_first = __builtin_amdgcn_readfirstlane(request_of(sm.pre, B, S0));
  const int r_last = __builtin_amdgcn_readfirstlane(request_of(sm.pre, B, S1 - 1));

  const size_t head_stride = (size_t)kPageSize * kHeadDim;          // elements per (page, KV head)
  const size_t page_stride = (size_t)a.num_kv_heads * head_stride;  // elements per page
  const uint16_t* kpool = a.k_pool + (size_t)g * head_stride;
  const uint16_t* vpool = a.v_pool + (size_t)g * head_stride;

  // Q of request r for this workgroup's heads, 8 bytes per thread t: column
  // t / 16 (query head g * G + column), dims 4 * (t % 16) .. + 3.
  auto load_q = [&](int t, int r) -> u32x2 {
    const int q_col = t >> 4, q_d0 = 4 * (t & 15);
    if (q_col >= G) return u32x2{};
    const uint16_t* p = a.q + ((size_t)r * a.num_qo_heads + g * G + q_col) * kHeadDim + q_d0;
    return *reinterpret_cast<const u32x2*>(p);
  };
  auto store_q = [&](int t, u32x2 x) {   // operand layout: lane (column, dims / 16), half (dims % 16) / 8
    const int q_col = t >> 4, q_d0 = 4 * (t & 15);
    uint8_t* dst = reinterpret_cast<uint8_t*>(&sm.u.run.q[(q_d0 & 15) >> 3][q_col + 16 * (q_d0 >> 4)]);
    *reinterpret_cast<u32x2*>(dst + 2 * (q_d0 & 7)) = x;
  };
  // page ids of a piece for this wave, lane l: the piece's page w + 4 l
  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  auto load_ids = [&](int l, int r, int a0, int n_pages, int group) -> int {
    const int i = wave + 4 * (64 * group + l);
    const int first = uni(sm.base[r] + (a0 - sm.pre[r]));
    return i < n_pages ? a.page_indices[first + i] : 0;
  };
  auto next_request = [&](int r) -> int {   // next request of the segment with pages in it, or -1
    for (int x = r + 1; x <= r_last; ++x)
      if (uni(sm.pre[x + 1]) > uni(sm.pre[x])) return x;
    return -1;
  };

  int ids_next = load_ids(lane, r_first, max(uni(sm.pre[r_first]), S0),
                          min(uni(sm.pre[r_first + 1]), S1) - max(uni(sm.pre[r_first]), S0), 0);

  for (int r = r_first; r >= 0; r = next_request(r)) {
    const int pr0 = uni(sm.pre[r]), pr1 = uni(sm.pre[r + 1]);
    const int a0 = max(pr0, S0), a1 = min(pr1, S1);
    const int n_pages = a1 - a0;
    const int n_k = uni(sm.nk[r]);
    const int lo_key = W > 0 ? max(0, n_k - W) : 0;
    const int pn0 = lo_key / kPageSize + (a0 - pr0);   // the request's page number of the piece's first page

    // lane-derived values, recomputed per piece from the lane id (see opaque)
    const int ln = opaque(__lane_id());
    const int t = 64 * wave + ln, col = ln & 15, grp = ln >> 4;
    const int lane_off = col * kHeadDim + 16 * grp;   // this lane's 32 bytes of a page block (K)
    // V in two contiguous kilobytes, 16 bytes a lane: keys ln / 8 and 8 + ln / 8,
    // chunk ln % 8 (whole runs per load stream faster than 32-byte pieces)
    const int v_key = ln >> 3, v_chunk = ln & 7;
    uint8_t* stage = sm.u.run.stage[wave];

    // Q of the piece's request (its load overlaps the page-id load issued
    // before: at the segment's start, or one piece ahead)
    store_q(t, load_q(t, r));
    int ids = ids_next;
    __syncthreads();                                   // Q staged; the LDS region is in the run layout
    const int r_after = next_request(r);
    if (r_after >= 0) {                                // prefetch the next piece's page ids
      const int b0 = uni(sm.pre[r_after]);            // it starts inside the segment
      ids_next = load_ids(ln, r_after, b0, min(uni(sm.pre[r_after + 1]), S1) - b0, 0);
    }
    // Q^T operands are read from LDS at every page (registers go to more waves)
    auto qop = [&](int half) -> bf16x8 { return __builtin_bit_cast(bf16x8, sm.u.run.q[half][ln]); };

    // key-domain streaming state (base 2) of this wave's pages of the piece
    float m = -kFloatMax, dsum = 0.f;
    f32x4 acc[4] = {};

    const int my_pages = n_pages > wave ? (n_pages - wave + kNW - 1) / kNW : 0;
    // One page in flight per wave (two measured slower: the extra registers
    // cost more waves than the deeper ring gains).
    u32x4 kc[2], vc[2];
    auto load_page = [&](int k) {      // this wave's k-th page of the piece (k < my_pages)
      const int id = __builtin_amdgcn_readlane(ids, k & 63);
      const size_t off = (size_t)id * page_stride;
      kc[0] = ldg16(kpool + off + lane_off);
      kc[1] = ldg16(kpool + off + lane_off + 8);
      vc[0] = ldg16(vpool + off + 8 * ln);
      vc[1] = ldg16(vpool + off + 8 * ln + 8 * kHeadDim);   // keys 8..15
    };
    if (my_pages > 0) load_page(0);
    for (int k = 0; k < my_pages; ++k) {
      const int pn = pn0 + wave + kNW * k;             // the request's page number
      f32x4 sc = {};
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[0]), qop(0), sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[1]), qop(1), sc, 0, 0, 0);
      // the slot is free once V is copied, so refill it now; past the wave's
      // last page it reloads that page (a cache hit), so that every path
      // issues the same loads
      const u32x4 v0r = vc[0], v1r = vc[1];
      if (((k + 1) & 63) == 0 && k + 1 < my_pages)   // next group of 64 ids (pieces over 256 pages)
        ids = load_ids(ln, r, a0, n_pages, (k + 1) >> 6);
      load_page(min(k + 1, my_pages - 1));
      const int key0 = pn * kPageSize + 4 * grp;
      // scaled scores (base 2) of the lane's four keys, -inf where not visible
      float s4[4];
      const bool full = pn * kPageSize >= lo_key && pn * kPageSize + kPageSize <= n_k;   // uniform
      if (full) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s4[i] = sc[i] * a.scale_log2;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int j = key0 + i;
          s4[i] = (j >= lo_key && j < n_k) ? sc[i] * a.scale_log2 : kNegInf;
        }
      }
      float tile_max = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
      tile_max = fmaxf(tile_max, shfl_xor_f32(tile_max, 16));
      tile_max = fmaxf(tile_max, shfl_xor_f32(tile_max, 32));
      const float m_new = fmaxf(m, tile_max);
      const float alpha = (m == m_new) ? 1.f : exp2_hw(m - m_new);
      m = m_new;
      dsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[db][i] *= alpha;
      float pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[i] = exp2_hw(s4[i] - m_new);
      const uint32_t p01 = pack_f16x2(pw[0], pw[1]);
      const uint32_t p23 = pack_f16x2(pw[2], pw[3]);
      dsum = add_f16x2(p23, add_f16x2(p01, dsum));
      const f16x4 pb = __builtin_bit_cast(f16x4, u32x2{p01, p23});

      // stage V (natural layout, swizzled); rows past the last key are zeroed
      // so that no stale or poisoned value can meet a zero weight
      u32x4 v0, v1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v0[e] = bf16x2_to_f16x2(v0r[e]);
        v1[e] = bf16x2_to_f16x2(v1r[e]);
      }
      if (pn * kPageSize + v_key >= n_k) v0 = u32x4{};
      if (pn * kPageSize + 8 + v_key >= n_k) v1 = u32x4{};
      *reinterpret_cast<u32x4*>(stage + page_swizzle(v_key, v_chunk)) = v0;
      *reinterpret_cast<u32x4*>(stage + page_swizzle(8 + v_key, v_chunk)) = v1;
      __asm__ volatile("" ::: "memory");
      // transposed read: lane (grp, j) addresses key 4*grp + j/4, dims 16*db + 4*(j%4)
      const int rkey = 4 * grp + (col >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int byte = page_swizzle(rkey, 2 * db + ((col & 3) >> 1)) + 8 * (col & 1);
        const i16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<__attribute__((address_space(3))) i16x4*>(reinterpret_cast<uintptr_t>(stage + byte)));
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, vt), pb, acc[db], 0, 0, 0);
      }
      __asm__ volatile("" ::: "memory");
    }
    // the four lanes of a column hold partial denominators
    dsum += shfl_xor_f32(dsum, 16);
    dsum += shfl_xor_f32(dsum, 32);

    // ---- merge the waves' states of this piece through LDS
    __syncthreads();                                    // staging and Q are free
    const int ln2 = opaque(__lane_id());               // (not held across the page loop)
    const int t2 = 64 * wave + ln2, col2 = ln2 & 15, grp2 = ln2 >> 4;
    if (grp2 == 0) {
      sm.u.merge.m[wave][col2] = m;
      sm.u.merge.d[wave][col2] = dsum;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
      *reinterpret_cast<f32x4*>(&sm.u.merge.o[wave][col2][16 * db + 4 * grp2]) = acc[db];
    __syncthreads();
    const bool whole = pr0 >= S0 && pr1 <= S1;          // the request lies in this segment
    const bool with_sink = a0 == pr0;                   // the piece holds the request's first page
    const int slot = s + r;
    for (int idx = t2; idx < G * kHeadDim; idx += kThreads) {
      const int c = idx / kHeadDim;
      const int d = idx % kHeadDim;
      const int h = g * G + c;
      // each wave's reference is finite (-FLT_MAX until its first key)
      float mx = -kFloatMax;
#pragma unroll
      for (int w = 0; w < kNW; ++w) mx = fmaxf(mx, sm.u.merge.m[w][c]);
      float den = 0.f, num = 0.f;
#pragma unroll
      for (int w = 0; w < kNW; ++w) {
        const float mw = sm.u.merge.m[w][c];
        const float wt = (mw == mx) ? 1.f : exp2_hw(mw - mx);
        den += wt * sm.u.merge.d[w][c];
        num += wt * sm.u.merge.o[w][c][d];
      }
      const float sink2 = (with_sink && a.sinks != nullptr) ? a.sinks[h] * kLog2e : kNegInf;
      float lse2;
      const float o = num * fold_sink(sink2, den > 0.f ? mx : kNegInf, den, &lse2);
      const float lse_nat = lse2 * kLn2;
      if (whole) {
        const size_t rh = (size_t)r * a.num_qo_heads + h;
        a.out[rh * kHeadDim + d] = to_bf16_bits(o);
        if (a.lse != nullptr && d == 0) a.lse[rh] = lse_nat;
      } else {
        const size_t sh = (size_t)slot * a.num_qo_heads + h;
        a.ws_o[sh * kHeadDim + d] = o;
        if (d == 0) a.ws_lse[sh] = lse_nat;
      }
    }
    __syncthreads();                                    // the merge area is free again
  }
}

// LSE merge of the partials in slots first .. first + cnt - 1 (cnt <= M) by
// one wave (lane = dimension): every load is issued before the first use
// (indices clamped to the last slot), so the wave waits one round trip.
template <int M>
__device__ __forceinline__ void merge_few(const float* lp, const float* op, size_t stride, int cnt, float& mx,
                                          float& den, float& num) {
  float l[M], o[M];
#pragma unroll
  for (int c = 0; c < M; ++c) {
    const size_t i = (size_t)min(c, cnt - 1);
    l[c] = lp[i * stride];
    o[c] = op[i * stride * kHeadDim];
  }
#pragma unroll
  for (int c = 0; c < M; ++c) {
    if (c >= cnt) l[c] = kNegInf;
    mx = fmaxf(mx, l[c]);
  }
  if (mx == kNegInf) return;
#pragma unroll
  for (int c = 0; c < M; ++c) {
    if (c >= cnt) break;
    const float wt = (l[c] == mx) ? 1.f : exp2_hw((l[c] - mx) * kLog2e);
    den += wt;
    num += wt * o[c];
  }
}

// Four (request, head) rows per workgroup of four waves, lane = dimension.
// Requests whose pieces lie in one segment were written by the decode kernel;
// a request without keys gets out = 0, lse = sink; the others merge their
// pieces' partials (the LSE merge of split partials).  When every row has at
// most 16 pieces each wave merges its own row with all loads issued first;
// otherwise (a long request can have a piece in almost every segment) each
// wave still takes its own row, its lanes split four ways over the pieces and
// sixteen ways over the dimensions: lane l merges pieces l / 16 + 4 k (sixteen
// a pass, every load issued first) on dimensions 4 (l % 16) .. + 3 into its
// own (maximum, sum, accumulator), and the four groups combine by shuffles.
constexpr int kMergeRows = 4;
constexpr int kMergeThreads = 64 * kMergeRows;

__global__ __launch_bounds__(kMergeThreads) void merge_balanced_kernel(BalancedArgs a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long rows = (long)a.batch * a.num_qo_heads;
  const long long T = a.ws_plan[a.batch], N = a.num_segments;
  const size_t stride = (size_t)a.num_qo_heads;                 // slots apart

  // every row of the workgroup: its first slot's offset, piece count
  // (0: nothing to merge) and kind
  int cnt[kMergeRows], s0v[kMergeRows];
  bool any_long = false;
#pragma unroll
  for (int j = 0; j < kMergeRows; ++j) {
    const long rh = (long)blockIdx.x * kMergeRows + j;
    cnt[j] = 0;
    s0v[j] = 0;
    if (rh >= rows) continue;
    const int r = (int)(rh / a.num_qo_heads);
    // the request's segments (-1: no key), clamped to [0, N) so that a plan
    // from another call cannot send the reads outside the workspace
    const int f = a.ws_seg[2 * r], l = a.ws_seg[2 * r + 1];
    if (f < 0) continue;
    const int s0 = max(0, f), s1 = min((int)N - 1, l);
    if (s0 >= s1) continue;                                      // written by the decode kernel
    cnt[j] = s1 - s0 + 1;
    s0v[j] = s0;
    any_long = any_long || cnt[j] > 16 || T < N;
  }
  // with more segments than pages some segments are empty (no workgroup
  // wrote their slots): only segments holding pages count
  auto held = [&](int j, int i) {
    const long long sg = s0v[j] + i;
    return T >= N || (sg * T) / N != ((sg + 1) * T) / N;
  };
  auto slot_ptrs = [&](int j, const float** lp, const float** op) {
    const long rh = (long)blockIdx.x * kMergeRows + j;
    const int r = (int)(rh / a.num_qo_heads), h = (int)(rh % a.num_qo_heads);
    *lp = a.ws_lse + (size_t)(s0v[j] + r) * stride + h;
    *op = a.ws_o + ((size_t)(s0v[j] + r) * stride + h) * kHeadDim + lane;
  };

  float mx = kNegInf, den = 0.f, num = 0.f;                       // of this wave's row
  if (!any_long) {
    if (cnt[wave] > 0) {
      const float *lp, *op;
      slot_ptrs(wave, &lp, &op);
      if (cnt[wave] <= 4) merge_few<4>(lp, op, stride, cnt[wave], mx, den, num);
      else if (cnt[wave] <= 8) merge_few<8>(lp, op, stride, cnt[wave], mx, den, num);
      else merge_few<16>(lp, op, stride, cnt[wave], mx, den, num);
    }
  } else {
    // wave = row; lane = (piece group lane / 16, dimension quad lane % 16):
    // the lane merges pieces lane / 16 + 4 k on dimensions 4 (lane % 16) .. + 3,
    // sixteen pieces a pass with every load issued first
    const int pg = lane >> 4, dq = lane & 15;
    float m_t = kNegInf, d_t = 0.f;
    f32x4 n_t = {0.f, 0.f, 0.f, 0.f};
    const int cw = cnt[wave];
    if (cw > 0) {
      const long rhw = (long)blockIdx.x * kMergeRows + wave;
      const int r = (int)(rhw / a.num_qo_heads), h = (int)(rhw % a.num_qo_heads);
      const float* lp = a.ws_lse + (size_t)(s0v[wave] + r) * stride + h;
      const f32x4* op4 = reinterpret_cast<const f32x4*>(a.ws_o + ((size_t)(s0v[wave] + r) * stride + h) * kHeadDim) + dq;
      for (int i0 = pg; i0 < cw; i0 += 4 * 16) {
        // a slot no workgroup wrote may hold anything (the kernels are built
        // assuming no NaN), so an entry past the row's pieces or in an empty
        // segment reads the row's first piece, always written, and weighs 0
        bool ok[16];
        float l[16];
        f32x4 o[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int i = i0 + 4 * u;
          ok[u] = i < cw && held(wave, i);
          const size_t ii = ok[u] ? (size_t)i : 0;
          l[u] = lp[ii * stride];
          o[u] = op4[ii * stride * (kHeadDim / 4)];
        }
        float m_new = m_t;
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (ok[u]) m_new = fmaxf(m_new, l[u]);
        if (m_new == kNegInf) continue;
        const float alpha = (m_t == m_new) ? 1.f : exp2_hw((m_t - m_new) * kLog2e);
        d_t *= alpha;
#pragma unroll
        for (int e = 0; e < 4; ++e) n_t[e] *= alpha;
        m_t = m_new;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          float wt = (l[u] == m_t) ? 1.f : exp2_hw((l[u] - m_t) * kLog2e);
          wt = ok[u] ? wt : 0.f;
          d_t += wt;
#pragma unroll
          for (int e = 0; e < 4; ++e) n_t[e] += wt * o[u][e];
        }
      }
    }
    // the four piece groups of the wave (lanes l, l ^ 16, l ^ 32, l ^ 48 hold
    // one dimension quad) combine by the LSE rule
    float mw = fmaxf(m_t, shfl_xor_f32(m_t, 16));
    mw = fmaxf(mw, shfl_xor_f32(mw, 32));
    const float sc = (m_t == kNegInf) ? 0.f : ((m_t == mw) ? 1.f : exp2_hw((m_t - mw) * kLog2e));
    float dw = d_t * sc;
    dw += shfl_xor_f32(dw, 16);
    dw += shfl_xor_f32(dw, 32);
    f32x4 nw;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      nw[e] = n_t[e] * sc;
      nw[e] += shfl_xor_f32(nw[e], 16);
      nw[e] += shfl_xor_f32(nw[e], 32);
    }
    if (cw > 0) {
      const long rhw = (long)blockIdx.x * kMergeRows + wave;
      if (pg == 0) {
        uint32_t hb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) hb[e] = to_bf16_bits(dw > 0.f ? nw[e] / dw : 0.f);
        *reinterpret_cast<u32x2*>(a.out + rhw * kHeadDim + 4 * dq) = u32x2{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
        if (a.lse != nullptr && dq == 0) a.lse[rhw] = dw > 0.f ? mw + __builtin_logf(dw) : mw;
      }
      return;
    }
  }

  // wave j writes row j
  const long rh = (long)blockIdx.x * kMergeRows + wave;
  if (rh >= rows) return;
  const int r = (int)(rh / a.num_qo_heads), h = (int)(rh % a.num_qo_heads);
  if (cnt[wave] == 0) {
    if (a.ws_seg[2 * r] >= 0) return;                            // written by the decode kernel
    const float sink2 = a.sinks != nullptr ? a.sinks[h] * kLog2e : kNegInf;   // no key: the sink alone
    float lse2;
    a.out[rh * kHeadDim + lane] = to_bf16_bits(0.f * fold_sink(sink2, kNegInf, 0.f, &lse2));
    if (a.lse != nullptr && lane == 0) a.lse[rh] = lse2 * kLn2;
    return;
  }
  a.out[rh * kHeadDim + lane] = to_bf16_bits(den > 0.f ? num / den : 0.f);
  if (a.lse != nullptr && lane == 0) a.lse[rh] = den > 0.f ? mx + __builtin_logf(den) : mx;
}

}  // namespace

hipError_t launch_decode_balanced(const BalancedArgs& a, hipStream_t stream) {
  const long wgs = (long)a.num_segments * a.num_kv_heads;
  if (wgs > 0) hipLaunchKernelGGL(decode_balanced_kernel, dim3((unsigned)wgs), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge_balanced(const BalancedArgs& a, hipStream_t stream) {
  const long rows = (long)a.batch * a.num_qo_heads;
  if (rows > 0)
    hipLaunchKernelGGL(merge_balanced_kernel, dim3((unsigned)((rows + kMergeRows - 1) / kMergeRows)),
                       dim3(kMergeThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sinkattn
