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
//        back transposed with ds_read_b64_tr_b16).  The Q^T operands are staged
//        in LDS once per workgroup.  The fp16 weights are taken relative to the
//        running key maximum; the sink is folded in at the end, which gives
//        exactly the state of the sink-seeded recurrence.
//   Each chunk's result is normalised by its own denominator and written as an
//   fp32 partial with its natural-log LSE, or, unsplit, as the bf16 output.
//   (Several query rows per request: verify.hip.)

#include "decode_common.hpp"
#include "device_common.hpp"
#include "kernel_args.hpp"

namespace sinkattn {
namespace {

constexpr int kPageBytes = kPageSize * kHeadDim * 2;  // one (page, KV head) block: 2 KiB
constexpr float kFloatMax = 3.402823466e38f;
// s_waitcnt operand: vector memory count 0, the other counters unconstrained
// (vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVm0 = 0x0F70;

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Byte offset of 16-byte chunk `chunk` of row `key` in a [16][64] bf16 page
// staged in LDS.  XOR-swizzling the chunk with the key spreads the rows of a
// transposed read over all banks.
__device__ __forceinline__ int page_swizzle(int key, int chunk) {
  return key * 128 + ((chunk ^ (key & 7)) << 4);
}

// LDS of a workgroup: per-wave V staging pages, then the Q^T operands
// (staged once, read every page: registers go to more waves); after the page
// loop the same bytes hold the cross-wave merge of the 16 columns.
template <int NW>
struct DecodeSmem {
  static constexpr int kStage = NW * kPageBytes;
  static constexpr int kQ = 2 * 64 * 16;
  static constexpr int kMerge = NW * 16 * (kHeadDim + 2) * 4;
  static constexpr int kBytes = kStage + kQ > kMerge ? kStage + kQ : kMerge;
};

// Waves per SIMD the kernel is held to (so that a register-count change
// cannot silently lower occupancy: a kernel that no longer fits spills, and
// the no-spill check of the build's tests fails).
constexpr int kDecodeWavesPerSimd = 7;

// NW waves per workgroup, one page in flight per wave.  Column j < G of the
// MFMAs is query head g * G + j, so the G heads of one KV head share every
// page load.
template <int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(kDecodeWavesPerSimd)))
void decode_paged_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[DecodeSmem<NW>::kBytes];

  const int lane = threadIdx.x & 63;
  // uniform per wave: keeps the page bookkeeping (and the page-id loads) scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;   // MFMA column (query head) or row (key) index
  const int grp = lane >> 4;   // 16-lane group
  const int S = a.num_splits;
  const int G = a.group;

  const DecodeUnit du = decode_unit<NW>(a);
  const int b = __builtin_amdgcn_readfirstlane(du.b);
  const int g = du.g, c = du.c;

  // the request's query row (in a mixed batch, requests with several rows
  // belong to the prefill kernel)
  int qrow = b;
  if (a.qo_indptr != nullptr) {
    const int r0 = a.qo_indptr[b];
    if (a.qo_indptr[b + 1] - r0 != 1) return;   // uniform: a prefill request, not ours
    qrow = r0;
  }
  qrow = __builtin_amdgcn_readfirstlane(qrow);

  // Keys this chunk attends to: the chunk's pages (ceil rule) intersected
  // with the row's window; the row sits at n_k - 1.
  const int n_k = __builtin_amdgcn_readfirstlane(du.n_k);
  const int lo_vis = a.window > 0 ? max(0, n_k - a.window) : 0;
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

  // Q^T operands of the score MFMA (column = head g * G + col, k = dims
  // 16 * grp + 8 * ks + e), loaded once by wave 0 into LDS and read from there
  // every page; columns past the group hold zeros.
  u32x4* const q_lds = reinterpret_cast<u32x4*>(smem + DecodeSmem<NW>::kStage);   // [2][64 lanes]
  if (wave == 0) {
    u32x4 x0 = {}, x1 = {};
    if (col < G) {
      const uint16_t* qp = a.q + ((size_t)qrow * a.num_qo_heads + g * G + col) * kHeadDim + 16 * grp;
      x0 = ldg16(qp);
      x1 = ldg16(qp + 8);
    }
    q_lds[lane] = x0;
    q_lds[64 + lane] = x1;
  }
  __syncthreads();
  auto qop = [&](int half) -> bf16x8 { return __builtin_bit_cast(bf16x8, q_lds[half * 64 + lane]); };

  // Key-domain streaming state (base 2): running key maximum, this lane's
  // part of the denominator, P.V accumulator.  The sink of chunk 0 is folded
  // in once the waves have merged (fold_sink), giving the state that the
  // recurrence seeded with (m, d) = (sink, 1) holds after the same keys.
  float m = -kFloatMax, dsum = 0.f;
  f32x4 acc[4] = {};

  const int32_t* pages = a.page_indices + __builtin_amdgcn_readfirstlane(du.page_base);
  const size_t head_stride = (size_t)kPageSize * kHeadDim;          // elements per (page, KV head)
  const size_t page_stride = (size_t)a.num_kv_heads * head_stride;  // elements per page
  const uint16_t* kpool = a.k_pool + (size_t)g * head_stride;
  const uint16_t* vpool = a.v_pool + (size_t)g * head_stride;
  const int lane_off = col * kHeadDim + 16 * grp;   // this lane's 32 bytes of a page block (K)
  // V is read in two contiguous kilobytes, 16 bytes a lane: keys lane / 8 and
  // 8 + lane / 8, chunk lane % 8 (a page's V goes through LDS anyway; whole
  // runs per load stream faster than the operand layout's 32-byte pieces)
  const int v_key = lane >> 3, v_chunk = lane & 7;
  uint8_t* stage = smem + wave * kPageBytes;

  // The wave's page ids arrive as vector loads, one lane per page, and each
  // page reads its id with readlane: no per-page scalar load and only one id
  // latency in front of the first page.  The wave's pages form groups of 64;
  // the ids of even groups live in ids0, of odd groups in ids1.  When
  // processing enters group g, the register of group g - 1 is reloaded with
  // group g + 1, 64 pages before its first use, so no id read on the common
  // path depends on a load of the same round.
  u32x4 kc[2], vc[2];
  int ids0 = lane < wp1 - wp0 ? pages[wp0 + lane] : 0;
  int ids1 = 64 + lane < wp1 - wp0 ? pages[wp0 + 64 + lane] : 0;
  // The id loads complete here and in each (rare) reload below, so that no
  // id register is ever seen as pending inside the page loop.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  int next_group = 1;                     // the group whose entry triggers the next reload
  auto page_id = [&](int p) -> int {      // p uniform, in group next_group or the one before
    const int r = p - wp0;
    return ((r >> 6) & 1) ? __builtin_amdgcn_readlane(ids1, r & 63) : __builtin_amdgcn_readlane(ids0, r & 63);
  };
  auto advance_ids = [&](int p) {         // p: the page being processed (uniform)
    const int gr = (p - wp0) >> 6;
    if (gr == next_group) {
      ++next_group;
      const int base = wp0 + 64 * (gr + 1);
      if (gr & 1) ids0 = base + lane < wp1 ? pages[base + lane] : 0;
      else ids1 = base + lane < wp1 ? pages[base + lane] : 0;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
  };
  auto load_page = [&](int p) {           // only while the run has pages
    if (p < wp1) {
      const size_t off = (size_t)page_id(p) * page_stride;
      const uint16_t* kp = kpool + off + lane_off;
      const uint16_t* vp = vpool + off + 8 * lane;
      kc[0] = ldg16(kp);
      kc[1] = ldg16(kp + 8);
      vc[0] = ldg16(vp);
      vc[1] = ldg16(vp + 8 * kHeadDim);   // keys 8..15
    }
  };
  load_page(wp0);

  // Waves streaming pages issue ahead of waves of other workgroups that are
  // loading their queries or merging their results (the loop is the part
  // whose loads must stay in flight).
  __builtin_amdgcn_s_setprio(3);
  for (int p = wp0; p < wp1; ++p) {
    // scores of page p
    f32x4 sc = {};
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[0]), qop(0), sc, 0, 0, 0);
    sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[1]), qop(1), sc, 0, 0, 0);
    // one page in flight: the slot is free once its registers are copied, so
    // refill it now
    const u32x4 v0r = vc[0], v1r = vc[1];
    advance_ids(p);
    load_page(p + 1);

    // scaled scores (base 2) of the lane's four keys, -inf where not visible
    const int key0 = p * kPageSize + 4 * grp;
    float s4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = key0 + i;
      s4[i] = (j >= t_lo && j <= t_hi - 1) ? sc[i] * a.scale_log2 : kNegInf;
    }
    // the running maximum moves with every page (the kernel is bound by the
    // page gathers, and this form holds fewer registers)
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
    // so that no stale or poisoned value can meet a zero weight.
    u32x4 v0, v1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v0[e] = bf16x2_to_f16x2(v0r[e]);
      v1[e] = bf16x2_to_f16x2(v1r[e]);
    }
    if (p * kPageSize + v_key >= n_k) v0 = u32x4{};
    if (p * kPageSize + 8 + v_key >= n_k) v1 = u32x4{};
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

  // merge the waves through LDS
  float* sm_m = reinterpret_cast<float*>(smem);
  float* sm_d = sm_m + NW * 16;
  float* sm_o = sm_d + NW * 16;   // [NW][16 columns][64 dims]
  __builtin_amdgcn_s_setprio(0);
  __syncthreads();                // the staging area is free
  if (grp == 0) {
    sm_m[wave * 16 + col] = m;
    sm_d[wave * 16 + col] = dsum;
  }
#pragma unroll
  for (int db = 0; db < 4; ++db)
    *reinterpret_cast<f32x4*>(sm_o + (wave * 16 + col) * kHeadDim + 16 * db + 4 * grp) = acc[db];
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * kHeadDim; idx += NW * 64) {
    const int j = idx / kHeadDim;
    const int d = idx % kHeadDim;
    const int h = g * G + j;
    // each wave's reference is finite (-FLT_MAX until its first visible key)
    float mx = -kFloatMax;
#pragma unroll
    for (int w = 0; w < NW; ++w) mx = fmaxf(mx, sm_m[w * 16 + j]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = sm_m[w * 16 + j];
      const float wt = (mw == mx) ? 1.f : exp2_hw(mw - mx);
      den += wt * sm_d[w * 16 + j];
      num += wt * sm_o[(w * 16 + j) * kHeadDim + d];
    }
    const float sink2 = (c == 0 && a.sinks != nullptr) ? a.sinks[h] * kLog2e : kNegInf;
    float lse2;
    // no visible key in the chunk: the key part is empty (d = 0)
    const float o = num * fold_sink(sink2, den > 0.f ? mx : kNegInf, den, &lse2);
    const float lse_nat = lse2 * kLn2;
    const size_t rh = (size_t)qrow * a.num_qo_heads + h;
    if (S == 1) {
      a.out[rh * kHeadDim + d] = to_bf16_bits(o);
      if (a.lse != nullptr && d == 0) a.lse[rh] = lse_nat;
    } else {
      a.o_part[(rh * S + c) * kHeadDim + d] = o;
      if (d == 0) a.lse_part[rh * S + c] = lse_nat;
    }
  }
}

// (row, head) pairs from which a merge launch packs four pairs into a wave.
constexpr long kMerge4MinPairs = 8192;

// One wave per (row, head); lane = output dimension.  With at most N chunks
// (N = 4, 8 or 16, the smallest that fits) every load -- the chunk LSEs and
// this lane's value of each partial -- is issued before the first use, so
// the wave waits for one memory round trip instead of one per chunk; more
// chunks take the plain loop.
template <int N>
__device__ __forceinline__ void merge_regs(const float* lp, const float* op, int S, float& mx,
                                           float& den, float& num) {
  float l[N], o[N];
#pragma unroll
  for (int c = 0; c < N; ++c) {   // index clamped to chunk S - 1: straight-line loads
    const int cc = min(c, S - 1);
    l[c] = lp[cc];
    o[c] = op[(long)cc * kHeadDim];
  }
#pragma unroll
  for (int c = 0; c < N; ++c) {
    if (c >= S) l[c] = kNegInf;
    mx = fmaxf(mx, l[c]);
  }
  if (mx == kNegInf) return;
#pragma unroll
  for (int c = 0; c < N; ++c) {   // chunks past S - 1 weigh exp2(-inf) = 0
    const float wt = (l[c] == mx) ? 1.f : exp2_hw((l[c] - mx) * kLog2e);
    den += wt;
    num += wt * o[c];
  }
}

__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const long rh = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rh >= (long)a.rows * a.num_heads) return;
  const int S = a.num_splits;
  const float* lp = a.lse_part + rh * S;
  const float* op = a.o_part + rh * S * kHeadDim + lane;
  float mx = kNegInf, den = 0.f, num = 0.f;
  if (S <= 4) {
    merge_regs<4>(lp, op, S, mx, den, num);
  } else if (S <= 8) {
    merge_regs<8>(lp, op, S, mx, den, num);
  } else if (S <= 16) {
    merge_regs<16>(lp, op, S, mx, den, num);
  } else {
    for (int c = 0; c < S; ++c) mx = fmaxf(mx, lp[c]);
    if (mx != kNegInf) {
      for (int c = 0; c < S; ++c) {
        const float l = lp[c];
        const float wt = (l == mx) ? 1.f : exp2_hw((l - mx) * kLog2e);
        den += wt;
        num += wt * op[(long)c * kHeadDim];
      }
    }
  }
  const float o = den > 0.f ? num / den : 0.f;
  a.out[rh * kHeadDim + lane] = to_bf16_bits(o);
  if (a.lse != nullptr && lane == 0) a.lse[rh] = den > 0.f ? mx + __builtin_logf(den) : mx;
}

// One (row, head) per sixteen lanes, four output dimensions a lane.  With at
// most N chunks (N = 4, 8 or 16, the smallest that fits) every load -- the
// chunk LSEs and this lane's four values of each partial -- is issued before
// the first use, so the wave waits for one memory round trip instead of one
// per chunk; more chunks take the plain loop.
template <int N>
__device__ __forceinline__ void merge_regs4(const float* lp, const f32x4* op, int S, float& mx,
                                           float& den, f32x4& num) {
  float l[N];
  f32x4 o[N];
#pragma unroll
  for (int c = 0; c < N; ++c) {   // index clamped to chunk S - 1: straight-line loads
    const int cc = min(c, S - 1);
    l[c] = lp[cc];
    o[c] = op[(long)cc * (kHeadDim / 4)];
  }
#pragma unroll
  for (int c = 0; c < N; ++c) {
    if (c >= S) l[c] = kNegInf;
    mx = fmaxf(mx, l[c]);
  }
  if (mx == kNegInf) return;
#pragma unroll
  for (int c = 0; c < N; ++c) {   // chunks past S - 1 weigh exp2(-inf) = 0 (no early exit:
                                  // the partials stay in registers)
    const float wt = (l[c] == mx) ? 1.f : exp2_hw((l[c] - mx) * kLog2e);
    den += wt;
#pragma unroll
    for (int e = 0; e < 4; ++e) num[e] += wt * o[c][e];
  }
}

// Four (row, head) pairs per wave, for launches with many pairs (one wave per
// pair left the verify batch's 21k pairs in three rounds of waves; with few
// pairs and many chunks, one pair per wave keeps more waves loading).
__global__ __launch_bounds__(256) void merge4_kernel(MergeArgs a) {
  const int lane = threadIdx.x & 63;
  const long rh = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
  if (rh >= (long)a.rows * a.num_heads) return;
  const int d0 = 4 * (lane & 15);
  const int S = a.num_splits;
  const float* lp = a.lse_part + rh * S;
  const f32x4* op = reinterpret_cast<const f32x4*>(a.o_part + rh * S * kHeadDim + d0);
  float mx = kNegInf, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  if (S <= 4) {
    merge_regs4<4>(lp, op, S, mx, den, num);
  } else if (S <= 8) {
    merge_regs4<8>(lp, op, S, mx, den, num);
  } else if (S <= 16) {
    merge_regs4<16>(lp, op, S, mx, den, num);
  } else {
    for (int c = 0; c < S; ++c) mx = fmaxf(mx, lp[c]);
    if (mx != kNegInf) {
      for (int c = 0; c < S; ++c) {
        const float l = lp[c];
        const float wt = (l == mx) ? 1.f : exp2_hw((l - mx) * kLog2e);
        den += wt;
        const f32x4 o = op[(long)c * (kHeadDim / 4)];
#pragma unroll
        for (int e = 0; e < 4; ++e) num[e] += wt * o[e];
      }
    }
  }
  uint32_t h[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = to_bf16_bits(den > 0.f ? num[e] / den : 0.f);
  *reinterpret_cast<u32x2*>(a.out + rh * kHeadDim + d0) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
  if (a.lse != nullptr && (lane & 15) == 0) a.lse[rh] = den > 0.f ? mx + __builtin_logf(den) : mx;
}

}  // namespace

// One-row decode: four waves per workgroup, one page in flight per wave (the
// launch shape measured fastest; deeper rings of pages in flight and eight
// waves per workgroup ran slower).
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const long units = (long)a.batch * a.num_kv_heads * a.num_splits;
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL(decode_paged_kernel<4>, dim3((unsigned)units), dim3(4 * 64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const long n = (long)a.rows * a.num_heads;
  if (n <= 0) return hipSuccess;
  if (n >= kMerge4MinPairs)
    hipLaunchKernelGGL(merge4_kernel, dim3((unsigned)((n + 15) / 16)), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sinkattn
