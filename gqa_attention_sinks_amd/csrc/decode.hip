// Paged-KV split decode with per-head attention sinks, and the LSE merge.
//
// Method: Perplexity blog "GPT-OSS on day 0" (French rendering "GPT-OSS au
// jour J"), section "Kernels for GPT-OSS > Sink attention": the streaming
// softmax keeps a running max m and a scale d; the sink is folded in by
// starting them at (sink, 1) instead of (-inf, 1), and when the KV sequence is
// split into blocks only the first block starts from the sink.  Paged KV and
// CPU-built page metadata: "Accelerating Sonar through speculation", section
// "Inference with speculative decoding".
//
// Work decomposition (gfx950, 64-lane waves):
//   workgroup = (request b, KV head g, chunk c); NW waves split the chunk's
//   pages into contiguous runs; at the end the waves merge through LDS.
//   Per page (16 keys x 64 dims = 2 KiB per KV head, contiguous in the pool):
//     S^T[16 keys x 16 heads] = K[16 x 64] . Q^T[64 x 16]  -> 2 x MFMA 16x16x32 bf16
//       (the G <= 16 query heads sharing KV head g are the MFMA columns; K goes
//        straight from HBM into the A operand, one 32-byte run per lane)
//     online softmax in base 2 on the accumulator (each lane: one head, 4 keys)
//     O^T[64 dims x 16 heads] += V^T . P^T                 -> 4 x MFMA 16x16x16 fp16
//       (P^T is the S^T accumulator converted in place to fp16; V is converted
//        to fp16 and staged in LDS in its natural [key][dim] layout, then read
//        back transposed with ds_read_b64_tr_b16).  The fp16 weights are taken
//        relative to the running key maximum; the sink is folded in at the end,
//        which gives exactly the state of the sink-seeded recurrence.
//   Each chunk's result is normalised by its own denominator and written as an
//   fp32 partial with its natural-log LSE, or, unsplit, as the bf16 output.

#include <stdio.h>
#include <stdlib.h>

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace sinkattn {
namespace {

constexpr int kPageBytes = kPageSize * kHeadDim * 2;  // one (page, KV head) block: 2 KiB

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Byte offset of 16-byte chunk `chunk` of row `key` in a [16][64] bf16 page
// staged in LDS.  XOR-swizzling the chunk with the key spreads the rows of a
// transposed read over all banks.
__device__ __forceinline__ int page_swizzle(int key, int chunk) {
  return key * 128 + ((chunk ^ (key & 7)) << 4);
}

template <int NW>
struct DecodeSmem {
  static constexpr int kStage = NW * kPageBytes;
  static constexpr int kMerge = NW * 16 * (kHeadDim + 2) * 4;
  static constexpr int kBytes = kStage > kMerge ? kStage : kMerge;
};

// Requests ranked by KV length (longest first), so that the longest chunks
// start first and the short ones fill the tail; only for batches up to this
// size (every workgroup ranks the batch itself).
constexpr int kRankMaxBatch = 256;

// Work unit of this workgroup: (request b, KV head g, chunk c), with the
// request's KV length and the offset of its page list.  Units are numbered
// request-major in rank order; within a request the KV heads come first, so
// consecutive workgroups (and XCDs) share a request's pages.  When ranking,
// the batch's lengths and page-list offsets are staged in LDS once, so the
// unit's own metadata costs no further dependent global load.
struct DecodeUnit { int b, g, c, n_k, page_base; };

template <int NW>
__device__ __forceinline__ DecodeUnit decode_unit(const DecodeArgs& a) {
  const int S = a.num_splits;
  int unit = blockIdx.x;
  DecodeUnit u;
  u.g = unit % a.num_kv_heads;
  unit /= a.num_kv_heads;
  u.c = unit % S;
  const int r = unit / S;
  if (a.batch <= kRankMaxBatch && a.batch > 1) {
    __shared__ int s_len[kRankMaxBatch];
    __shared__ int s_ptr[kRankMaxBatch];
    __shared__ int s_req;
    for (int i = threadIdx.x; i < a.batch; i += NW * 64) {
      s_len[i] = a.kv_len[i];
      s_ptr[i] = a.page_indptr[i];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < a.batch; i += NW * 64) {
      const int li = s_len[i];
      int rank = 0;
      for (int j = 0; j < a.batch; ++j) {
        const int lj = s_len[j];
        rank += (lj > li) || (lj == li && j < i);
      }
      if (rank == r) s_req = i;   // ranks are a permutation: exactly one writer
    }
    __syncthreads();
    u.b = s_req;
    u.n_k = s_len[u.b];
    u.page_base = s_ptr[u.b];
  } else {
    u.b = r;
    u.n_k = a.kv_len[r];
    u.page_base = a.page_indptr[r];
  }
  return u;
}

// PF: pages in flight per wave (a ring of register buffers; the loop is
// unrolled by PF so the ring slots are static).
template <int NW, int PF>
__global__ __launch_bounds__(NW * 64) void decode_paged_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[DecodeSmem<NW>::kBytes];

  const int lane = threadIdx.x & 63;
  // uniform per wave: keeps the page bookkeeping (and the page-id loads) scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;   // MFMA column (query head) or row (key) index
  const int grp = lane >> 4;   // 16-lane group
  const int S = a.num_splits;

  const DecodeUnit du = decode_unit<NW>(a);
  const int b = __builtin_amdgcn_readfirstlane(du.b);
  const int g = du.g, c = du.c;

  int qrow = b;
  if (a.qo_indptr != nullptr) {
    const int r0 = a.qo_indptr[b];
    if (a.qo_indptr[b + 1] - r0 != 1) return;   // a prefill request: not ours
    qrow = r0;
  }

  // Keys this chunk attends to: chunk pages (ceil rule) intersected with the
  // causal / window range of the query at position n_k - 1.
  const int n_k = __builtin_amdgcn_readfirstlane(du.n_k);
  const int pos = n_k - 1;
  const int lo_vis = a.window > 0 ? max(0, pos - a.window + 1) : 0;
  const int n_pages = (n_k + kPageSize - 1) / kPageSize;
  const int ppc = (n_pages + S - 1) / S;
  const int cp0 = min(c * ppc, n_pages);
  const int cp1 = min((c + 1) * ppc, n_pages);
  const int t_lo = max(cp0 * kPageSize, lo_vis);
  const int t_hi = min(cp1 * kPageSize, n_k);
  const int pg0 = t_lo / kPageSize;
  const int pg1 = t_hi > t_lo ? (t_hi + kPageSize - 1) / kPageSize : pg0;
  const int per_wave = (pg1 - pg0 + NW - 1) / NW;
  const int wp0 = min(pg0 + wave * per_wave, pg1);
  const int wp1 = min(wp0 + per_wave, pg1);

  const int head = g * a.group + col;
  const bool head_ok = col < a.group;

  // Q^T operand of the score MFMA: column = head, k = dims 16*grp + 8*ks + e.
  bf16x8 q0 = {}, q1 = {};
  if (head_ok) {
    const uint16_t* qp = a.q + ((size_t)qrow * a.num_qo_heads + head) * kHeadDim + 16 * grp;
    q0 = __builtin_bit_cast(bf16x8, ldg16(qp));
    q1 = __builtin_bit_cast(bf16x8, ldg16(qp + 8));
  }

  // Key-domain streaming state (base 2): running key max, this lane's part of
  // the denominator, P.V accumulator.  The sink of chunk 0 is folded in once
  // the waves have merged (fold_sink), giving the state that the recurrence
  // seeded with (m, d) = (sink, 1) holds after the same keys.
  float m = kNegInf, dsum = 0.f;
  f32x4 acc[4] = {};

  const int32_t* pages = a.page_indices + __builtin_amdgcn_readfirstlane(du.page_base);
  const size_t head_stride = (size_t)kPageSize * kHeadDim;          // elements per (page, KV head)
  const size_t page_stride = (size_t)a.num_kv_heads * head_stride;  // elements per page
  const uint16_t* kpool = a.k_pool + (size_t)g * head_stride;
  const uint16_t* vpool = a.v_pool + (size_t)g * head_stride;
  const int lane_off = col * kHeadDim + 16 * grp;   // this lane's 32 bytes of a page block
  uint8_t* stage = smem + wave * kPageBytes;

  // Ring of PF pages in flight: slot u holds page lp + u of the current
  // round.  The wave's page ids arrive as one vector load (lane i holds the
  // id of page wp0 + 64*k + i, reloaded every 64 pages), issued together
  // with Q, and each step reads its id with readlane: no per-page scalar load
  // and only one id latency in front of the first page.
  u32x4 kc[PF][2], vc[PF][2];
  int id_vec = lane < wp1 - wp0 ? pages[wp0 + lane] : 0;
  int id_base = wp0;                      // page index of id_vec's lane 0
  auto page_id = [&](int p) -> int {      // p uniform, wp0 <= p < id_base + 64
    return __builtin_amdgcn_readlane(id_vec, p - id_base);
  };
  auto load_page = [&](int u, int p) {
    if (p < wp1) {
      if (p - id_base >= 64) {            // uniform: next 64 ids
        id_base += 64;
        id_vec = id_base + lane < wp1 ? pages[id_base + lane] : 0;
      }
      const size_t off = (size_t)page_id(p) * page_stride;
      const uint16_t* kp = kpool + off + lane_off;
      const uint16_t* vp = vpool + off + lane_off;
      kc[u][0] = ldg16(kp);
      kc[u][1] = ldg16(kp + 8);
      vc[u][0] = ldg16(vp);
      vc[u][1] = ldg16(vp + 8);
    }
  };
#pragma unroll
  for (int u = 0; u < PF; ++u) load_page(u, wp0 + u);

  for (int lp = wp0; lp < wp1; lp += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int p = lp + u;
      if (p >= wp1) break;
      // scores of page p (ring slot u)
      f32x4 sc = {};
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[u][0]), q0, sc, 0, 0, 0);
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[u][1]), q1, sc, 0, 0, 0);
      const u32x4 v0r = vc[u][0], v1r = vc[u][1];
      // the slot is free once its registers are consumed: refill it
      load_page(u, p + PF);

      float s4[4];
      float tile_max = kNegInf;
      const int key0 = p * kPageSize + 4 * grp;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = key0 + i;
        const bool vis = j >= t_lo && j < t_hi;
        s4[i] = vis ? sc[i] * a.scale_log2 : kNegInf;
        tile_max = fmaxf(tile_max, s4[i]);
      }
      tile_max = fmaxf(tile_max, shfl_xor_f32(tile_max, 16));
      tile_max = fmaxf(tile_max, shfl_xor_f32(tile_max, 32));
      const float m_new = fmaxf(m, tile_max);
      const float alpha = (m == m_new) ? 1.f : exp2_hw(m - m_new);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      m = m_new;
      dsum *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[db][i] *= alpha;

      float pw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pw[i] = exp2_hw(s4[i] - m_use);
      const uint32_t p01 = pack_f16x2(pw[0], pw[1]);
      const uint32_t p23 = pack_f16x2(pw[2], pw[3]);
      dsum = add_f16x2(p23, add_f16x2(p01, dsum));
      const f16x4 pb = __builtin_bit_cast(f16x4, u32x2{p01, p23});

      // stage V (natural layout, swizzled); rows past the last key are zeroed
      // so that no stale or poisoned value can meet a zero weight.
      u32x4 v0, v1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v0[e] = bf16x2_to_f16x2(v0r[e]);
        v1[e] = bf16x2_to_f16x2(v1r[e]);
      }
      if (p * kPageSize + col >= n_k) { v0 = u32x4{}; v1 = u32x4{}; }
      *reinterpret_cast<u32x4*>(stage + page_swizzle(col, 2 * grp)) = v0;
      *reinterpret_cast<u32x4*>(stage + page_swizzle(col, 2 * grp + 1)) = v1;
      __asm__ volatile("" ::: "memory");
      // transposed read: lane (grp, j) addresses key 4*grp + j/4, dims 16*db + 4*(j%4)
      const int rkey = 4 * grp + (col >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int byte = page_swizzle(rkey, 2 * db + ((col & 3) >> 1)) + 8 * (col & 1);
        const i16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<__attribute__((address_space(3))) i16x4*>(
                reinterpret_cast<uintptr_t>(stage + byte)));
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, vt), pb, acc[db], 0, 0, 0);
      }
      __asm__ volatile("" ::: "memory");
    }
  }

  // the four lanes of a head hold partial denominators
  dsum += shfl_xor_f32(dsum, 16);
  dsum += shfl_xor_f32(dsum, 32);

  // merge the waves through LDS
  __syncthreads();
  float* sm_m = reinterpret_cast<float*>(smem);
  float* sm_d = sm_m + NW * 16;
  float* sm_o = sm_d + NW * 16;   // [NW][16 heads][64 dims]
  if (grp == 0) {
    sm_m[wave * 16 + col] = m;
    sm_d[wave * 16 + col] = dsum;
  }
#pragma unroll
  for (int db = 0; db < 4; ++db)
    *reinterpret_cast<f32x4*>(sm_o + (wave * 16 + col) * kHeadDim + 16 * db + 4 * grp) = acc[db];
  __syncthreads();

  for (int idx = threadIdx.x; idx < a.group * kHeadDim; idx += NW * 64) {
    const int hh = idx / kHeadDim;
    const int d = idx % kHeadDim;
    const int h = g * a.group + hh;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, sm_m[w * 16 + hh]);
    float den = 0.f, num = 0.f;
    if (mx != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = sm_m[w * 16 + hh];
        const float wt = (mw == mx) ? 1.f : exp2_hw(mw - mx);
        den += wt * sm_d[w * 16 + hh];
        num += wt * sm_o[(w * 16 + hh) * kHeadDim + d];
      }
    }
    const float sink2 = (c == 0 && a.sinks != nullptr) ? a.sinks[h] * kLog2e : kNegInf;
    float lse2;
    const float o = num * fold_sink(sink2, mx, den, &lse2);
    const float lse_nat = lse2 * kLn2;
    if (S == 1) {
      a.out[((size_t)qrow * a.num_qo_heads + h) * kHeadDim + d] = to_bf16_bits(o);
      if (a.lse != nullptr && d == 0) a.lse[(size_t)qrow * a.num_qo_heads + h] = lse_nat;
    } else {
      const size_t rh = (size_t)b * a.num_qo_heads + h;
      a.o_part[(rh * S + c) * kHeadDim + d] = o;
      if (d == 0) a.lse_part[rh * S + c] = lse_nat;
    }
  }
}

// One wave per (row, head); lane = output dimension.
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const long rh = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rh >= (long)a.rows * a.num_heads) return;
  const int S = a.num_splits;
  const float* lp = a.lse_part + rh * S;
  const float* op = a.o_part + rh * S * kHeadDim + lane;
  float mx = kNegInf;
  for (int c = 0; c < S; ++c) mx = fmaxf(mx, lp[c]);
  float den = 0.f, num = 0.f;
  if (mx != kNegInf) {
    for (int c = 0; c < S; ++c) {
      const float l = lp[c];
      const float wt = (l == mx) ? 1.f : exp2_hw((l - mx) * kLog2e);
      den += wt;
      num += wt * op[(long)c * kHeadDim];
    }
  }
  const float o = den > 0.f ? num / den : 0.f;
  a.out[rh * kHeadDim + lane] = to_bf16_bits(o);
  if (a.lse != nullptr && lane == 0) a.lse[rh] = den > 0.f ? mx + __builtin_logf(den) : mx;
}

}  // namespace

// Launch shapes: (waves per workgroup, pages in flight per wave).
// SINKATTN_DECODE_SHAPE ("4x2", "8x1", ...) overrides the default for tuning
// runs.
struct DecodeShape { int nw, pf; };

static DecodeShape decode_shape() {
  static const DecodeShape shape = [] {
    DecodeShape d{4, 1};
    if (const char* e = getenv("SINKATTN_DECODE_SHAPE")) {
      int nw = 0, pf = 0;
      if (sscanf(e, "%dx%d", &nw, &pf) == 2) d = DecodeShape{nw, pf};
    }
    return d;
  }();
  return shape;
}

template <int NW, int PF>
static void launch_shape(const DecodeArgs& a, long units, hipStream_t stream) {
  hipLaunchKernelGGL((decode_paged_kernel<NW, PF>), dim3((unsigned)units), dim3(NW * 64), 0, stream, a);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const long units = (long)a.batch * a.num_kv_heads * a.num_splits;
  if (units <= 0) return hipSuccess;
  const DecodeShape d = decode_shape();
  if (d.nw == 4 && d.pf == 1) launch_shape<4, 1>(a, units, stream);
  else if (d.nw == 4 && d.pf == 3) launch_shape<4, 3>(a, units, stream);
  else if (d.nw == 4 && d.pf == 4) launch_shape<4, 4>(a, units, stream);
  else if (d.nw == 8 && d.pf == 1) launch_shape<8, 1>(a, units, stream);
  else if (d.nw == 8 && d.pf == 2) launch_shape<8, 2>(a, units, stream);
  else if (d.nw == 2 && d.pf == 4) launch_shape<2, 4>(a, units, stream);
  else launch_shape<4, 2>(a, units, stream);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const long n = (long)a.rows * a.num_heads;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sinkattn
