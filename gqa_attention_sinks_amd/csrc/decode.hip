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
//        running key maximum (one row) or to a reference that moves only when
//        a weight would overflow (several rows); the sink is folded in at the
//        end, which gives exactly the state of the sink-seeded recurrence.
//   Each chunk's result is normalised by its own denominator and written as an
//   fp32 partial with its natural-log LSE, or, unsplit, as the bf16 output.
//   Several query rows per request (a speculative verify step, "Accelerating
//   Sonar through speculation", section "Speculative decoding"): the MFMA
//   columns are (row, head) pairs, up to four 16-column blocks that share
//   every page load, each column masked at its own causal position.

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace sinkattn {
namespace {

constexpr int kPageBytes = kPageSize * kHeadDim * 2;  // one (page, KV head) block: 2 KiB
// fp16 weights are taken against a reference that moves only when some weight
// would exceed this (fp16 keeps them finite, the rescale stays rare)
constexpr float kWeightLimit = 16384.f;
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
// loop the same bytes hold the cross-wave merge of one 16-column block.
template <int NW, int NB>
struct DecodeSmem {
  static constexpr int kStage = NW * kPageBytes;
  static constexpr int kQ = NB * 2 * 64 * 16;
  static constexpr int kMerge = NW * 16 * (kHeadDim + 2) * 4;
  static constexpr int kBytes = kStage + kQ > kMerge ? kStage + kQ : kMerge;
};

// Requests ranked by KV length (longest first), so that the longest chunks
// start first and the short ones fill the tail; only for batches up to this
// size (every workgroup ranks the batch itself).  Padding entries of -1 never
// outrank a real request (kv_len >= 0).
constexpr int kRankMaxBatch = 256;
// Under a window up to this long every request's work is about the same, and
// ranking would only cost time.
constexpr int kRankMinWindow = 2048;

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
  if (a.batch <= kRankMaxBatch && a.batch > 1 && (a.window == 0 || a.window > kRankMinWindow)) {
    __shared__ __attribute__((aligned(16))) int s_len[kRankMaxBatch];
    __shared__ int s_ptr[kRankMaxBatch];
    __shared__ int s_req;
    const int nb4 = (a.batch + 3) & ~3;   // padded to whole int4s with -1 (ranks below every length)
    for (int i = threadIdx.x; i < nb4; i += NW * 64) {
      s_len[i] = i < a.batch ? a.kv_len[i] : -1;
      if (i < a.batch) s_ptr[i] = a.page_indptr[i];
    }
    __syncthreads();
    for (int i = threadIdx.x; i < a.batch; i += NW * 64) {
      const int li = s_len[i];
      int rank = 0;
      for (int j = 0; j < nb4; j += 4) {   // four lengths per LDS read (same address for the wave)
        const int4 l4 = *reinterpret_cast<const int4*>(&s_len[j]);
        rank += (l4.x > li) || (l4.x == li && j < i);
        rank += (l4.y > li) || (l4.y == li && j + 1 < i);
        rank += (l4.z > li) || (l4.z == li && j + 2 < i);
        rank += (l4.w > li) || (l4.w == li && j + 3 < i);
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

// Waves per SIMD each variant is held to (so that a register-count change
// cannot silently lower occupancy; a variant that no longer fits spills, and
// the no-spill check of the build's tests fails): one page in flight with one
// row fits seven; the multi-row variants hold about 80, 110 and 160 VGPRs for
// one, two and four column blocks.
constexpr int decode_waves_per_simd(int PF, int NB, bool MULTI) {
  return PF > 1 ? 1 : !MULTI ? 7 : NB == 1 ? 6 : NB == 2 ? 4 : 3;
}

// PF: pages in flight per wave (a ring of register buffers; the loop is
// unrolled by PF so the ring slots are static).  NB: 16-column blocks of the
// MFMAs.  Column j of the blocks is (query row j / G, query head j % G) of
// the request, so the G heads of one KV head share every page load; one
// query row per request fills G of the 16 columns of one block, several rows
// (MULTI: the rows of qo_indptr, as in a speculative verify step) fill up to
// NB blocks, each column with its own causal limit.  MASK (with MULTI): a
// bit-packed custom mask per request (a draft tree) decides which keys each
// row sees, instead of the causal rule.
template <int NW, int PF, int NB, bool MULTI, bool MASK>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(decode_waves_per_simd(PF, NB, MULTI))))
void decode_paged_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[DecodeSmem<NW, NB>::kBytes];

  const int lane = threadIdx.x & 63;
  // uniform per wave: keeps the page bookkeeping (and the page-id loads) scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;   // MFMA column (query row and head) or row (key) index
  const int grp = lane >> 4;   // 16-lane group
  const int S = a.num_splits;
  const int G = a.group;

  const DecodeUnit du = decode_unit<NW>(a);
  const int b = __builtin_amdgcn_readfirstlane(du.b);
  const int g = du.g, c = du.c;

  // the request's first query row and its number of rows
  int qrow = b, n_q = 1;
  if (MULTI) {
    const int r0 = a.qo_indptr[b];
    qrow = r0;
    n_q = min(a.qo_indptr[b + 1] - r0, a.max_rows);
    if (n_q < 1) return;                          // uniform: an empty request
  } else if (a.qo_indptr != nullptr) {
    const int r0 = a.qo_indptr[b];
    if (a.qo_indptr[b + 1] - r0 != 1) return;   // a prefill request: not ours
    qrow = r0;
  }
  qrow = __builtin_amdgcn_readfirstlane(qrow);
  n_q = __builtin_amdgcn_readfirstlane(n_q);
  // column blocks this request fills (the others are skipped: uniform branches)
  const int nb_used = MULTI ? (G * n_q + 15) / 16 : 1;

  // Keys this chunk attends to: chunk pages (ceil rule) intersected with the
  // union of the rows' causal / window ranges; row t sits at n_k - n_q + t.
  const int n_k = __builtin_amdgcn_readfirstlane(du.n_k);
  const int lo_vis = (!MASK && a.window > 0) ? max(0, n_k - n_q - a.window + 1) : 0;
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
  // keys every row of the request sees: [full_lo, full_hi] within the chunk
  const int full_lo = a.window > 0 ? max(t_lo, n_k - a.window) : t_lo;
  const int full_hi = min(t_hi - 1, n_k - n_q);

  // This lane's columns: Q^T operands of the score MFMA (column = (row, head),
  // k = dims 16*grp + 8*ks + e), loaded once by wave 0 into LDS and read from
  // there every page, and the keys of the chunk each column may see,
  // [v_lo, v_hi] (with several rows: its own causal / window range; a mask,
  // where given, decides inside it).
  int v_lo[NB], v_hi[NB];
  int c_bit[NB];   // MASK: bit offset of the column's mask row in the request's mask (-1: no row)
  u32x4* const q_lds = reinterpret_cast<u32x4*>(smem + DecodeSmem<NW, NB>::kStage);   // [NB][2][64 lanes]
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int j = 16 * nb + col;
    const int t = j / G;
    const int head = g * G + (j - t * G);
    if (wave == 0) {
      u32x4 x0 = {}, x1 = {};
      if (t < n_q) {
        const uint16_t* qp = a.q + ((size_t)(qrow + t) * a.num_qo_heads + head) * kHeadDim + 16 * grp;
        x0 = ldg16(qp);
        x1 = ldg16(qp + 8);
      }
      q_lds[(nb * 2) * 64 + lane] = x0;
      q_lds[(nb * 2 + 1) * 64 + lane] = x1;
    }
    const int c_pos = n_k - n_q + t;
    const int c_lo = a.window > 0 ? c_pos - a.window + 1 : 0;
    v_lo[nb] = MULTI && !MASK ? max(t_lo, c_lo) : t_lo;
    v_hi[nb] = MULTI && !MASK ? min(t_hi - 1, c_pos) : t_hi - 1;
    c_bit[nb] = t < n_q ? t * n_k : -1;
  }
  __syncthreads();
  auto qop = [&](int nb, int half) -> bf16x8 {
    return __builtin_bit_cast(bf16x8, q_lds[(nb * 2 + half) * 64 + lane]);
  };
  // the request's mask: row t, key j is bit t * n_k + j (little-endian bytes)
  const uint8_t* mbytes = MASK ? a.custom_mask + a.mask_indptr[b] : nullptr;

  // Key-domain streaming state (base 2) per column block: running key max,
  // this lane's part of the denominator, P.V accumulator.  The sink of chunk
  // 0 is folded in once the waves have merged (fold_sink), giving the state
  // that the recurrence seeded with (m, d) = (sink, 1) holds after the same
  // keys.
  float m[NB], dsum[NB];
  f32x4 acc[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m[nb] = -kFloatMax;
    dsum[nb] = 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db) acc[nb][db] = f32x4{};
  }

  const int32_t* pages = a.page_indices + __builtin_amdgcn_readfirstlane(du.page_base);
  const size_t head_stride = (size_t)kPageSize * kHeadDim;          // elements per (page, KV head)
  const size_t page_stride = (size_t)a.num_kv_heads * head_stride;  // elements per page
  const uint16_t* kpool = a.k_pool + (size_t)g * head_stride;
  const uint16_t* vpool = a.v_pool + (size_t)g * head_stride;
  const int lane_off = col * kHeadDim + 16 * grp;   // this lane's 32 bytes of a page block
  uint8_t* stage = smem + wave * kPageBytes;

  // Ring of PF pages in flight: slot u holds page lp + u of the current
  // round.  The wave's page ids arrive as vector loads, one lane per page, and
  // each step reads its id with readlane: no per-page scalar load and only one
  // id latency in front of the first page.  The wave's pages form groups of
  // 64; the ids of even groups live in ids0, of odd groups in ids1.  When
  // processing enters group g, the register of group g - 1 is reloaded with
  // group g + 1, 64 pages before its first use, so no id read on the common
  // path depends on a load of the same round.
  //
  // With several pages in flight every path through the page loop must issue
  // the same loads in the same order, or the compiler's count of loads in
  // flight turns conservative and waits for all of them before each page:
  // past the end of the wave's run a slot is refilled with the run's last
  // page again (a cache hit) rather than skipped.
  u32x4 kc[PF][2], vc[PF][2];
  uint32_t mk[PF][NB];   // MASK: this lane's four mask bits per column block
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
    const int g = (p - wp0) >> 6;
    if (g == next_group) {
      ++next_group;
      const int base = wp0 + 64 * (g + 1);
      if (g & 1) ids0 = base + lane < wp1 ? pages[base + lane] : 0;
      else ids1 = base + lane < wp1 ? pages[base + lane] : 0;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
  };
  auto load_page = [&](int u, int p) {   // several in flight: only while the run has pages
    if (PF > 1 || p < wp1) {
      const int pc = PF > 1 ? min(p, wp1 - 1) : p;
      const size_t off = (size_t)page_id(pc) * page_stride;
      const uint16_t* kp = kpool + off + lane_off;
      const uint16_t* vp = vpool + off + lane_off;
      kc[u][0] = ldg16(kp);
      kc[u][1] = ldg16(kp + 8);
      vc[u][0] = ldg16(vp);
      vc[u][1] = ldg16(vp + 8);
      if (MASK) {
        // keys key0 .. key0 + 3 of this lane; the bytes read stop at the
        // request's last key, so they stay inside its mask
        const int key0 = pc * kPageSize + 4 * grp;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          mk[u][nb] = 0;
          if (nb < nb_used && c_bit[nb] >= 0 && key0 < n_k) {
            const int bit0 = c_bit[nb] + key0;
            const int bit1 = c_bit[nb] + min(key0 + 3, n_k - 1);
            uint32_t w = mbytes[bit0 >> 3];
            if ((bit1 >> 3) != (bit0 >> 3)) w |= (uint32_t)mbytes[bit1 >> 3] << 8;
            mk[u][nb] = (w >> (bit0 & 7)) & 0xFu;
          }
        }
      }
    }
  };
  if (PF == 1 || wp0 < wp1) {
#pragma unroll
    for (int u = 0; u < PF; ++u) load_page(u, wp0 + u);
  }

  // One page: ring slot u holds page p.  With several pages in flight, full
  // rounds of PF pages run in the main loop and the last, partial round after
  // it, so that every path through the loop body leaves the slots' loads in
  // flight in the same order.
  auto page_step = [&](const int u, const int p) __attribute__((always_inline)) {
      // scores of page p (ring slot u), every column block
      f32x4 sc[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        sc[nb] = f32x4{};
        if (nb >= nb_used) continue;
        sc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[u][0]), qop(nb, 0), sc[nb], 0, 0, 0);
        sc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[u][1]), qop(nb, 1), sc[nb], 0, 0, 0);
      }
      uint32_t mcur[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) mcur[nb] = MASK ? mk[u][nb] : 0u;
      // One page in flight: the slot is free once its registers are copied,
      // so refill it now.  Several: refill after V is staged (no copy, and no
      // wait on the other slots' loads).
      u32x4 v0r, v1r;
      if constexpr (PF == 1) {
        v0r = vc[u][0];
        v1r = vc[u][1];
        advance_ids(p);
        load_page(u, p + PF);
      }

      const int key0 = p * kPageSize + 4 * grp;
      // uniform: every key of the page visible to every column (no per-key test)
      const bool page_full = !MASK && p * kPageSize >= full_lo && p * kPageSize + kPageSize - 1 <= full_hi;
      // with a mask: the page inside the chunk and every key visible to every
      // real column of the block (a draft tree shows its rows the whole
      // context, so this is every page but the last few)
      const bool page_in = MASK && p * kPageSize >= t_lo && p * kPageSize + kPageSize - 1 <= t_hi - 1;
      auto block_full = [&](int nb) -> bool {
        if constexpr (!MASK) return page_full;
        return page_in && __builtin_amdgcn_ballot_w64(c_bit[nb] >= 0 && mcur[nb] != 0xFu) == 0;
      };
      f16x4 pb[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        pb[nb] = f16x4{};
        if (nb >= nb_used) continue;
        auto visible = [&](int i) -> bool {
          const int j = key0 + i;
          bool vis = j >= v_lo[nb] && j <= v_hi[nb];
          if (MASK) vis = vis && ((mcur[nb] >> i) & 1u);
          return vis;
        };
        // scaled scores (base 2) of the lane's four keys, -inf where not visible
        auto masked_scores = [&](float (&s4)[4]) {
#pragma unroll
          for (int i = 0; i < 4; ++i) s4[i] = visible(i) ? sc[nb][i] * a.scale_log2 : kNegInf;
        };
        float pw[4];
        if constexpr (MULTI) {
          // Weights against the current reference m (the same arithmetic on
          // every visible key, whichever the path).  A weight above the limit
          // means a key well above the reference (always on a wave's first
          // visible page, m starting at -FLT_MAX): move the reference to the
          // column maxima, rescale, and redo the weights.
#pragma unroll
          for (int i = 0; i < 4; ++i) pw[i] = exp2_hw(__builtin_fmaf(sc[nb][i], a.scale_log2, -m[nb]));
          if (!block_full(nb)) {   // uniform: one branch per block, selects inside
#pragma unroll
            for (int i = 0; i < 4; ++i) pw[i] = visible(i) ? pw[i] : 0.f;
          }
          const float pmax = fmaxf(fmaxf(pw[0], pw[1]), fmaxf(pw[2], pw[3]));
          if (__builtin_amdgcn_ballot_w64(pmax > kWeightLimit) != 0) {
            // the keys that can move the reference are those with a nonzero
            // weight: a hidden key's weight is 0, and one that underflowed
            // lies far below the reference
            float s4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) s4[i] = pw[i] > 0.f ? sc[nb][i] * a.scale_log2 : kNegInf;
            float tile_max = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
            tile_max = fmaxf(tile_max, shfl_xor_f32(tile_max, 16));
            tile_max = fmaxf(tile_max, shfl_xor_f32(tile_max, 32));
            const float m_new = fmaxf(m[nb], tile_max);
            const float alpha = exp2_hw(m[nb] - m_new);
            m[nb] = m_new;
            dsum[nb] *= alpha;
#pragma unroll
            for (int db = 0; db < 4; ++db)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[nb][db][i] *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) pw[i] = exp2_hw(s4[i] - m_new);
          }
        } else {
          // one row: the running maximum moves with every page (the kernel is
          // bound by the page gathers, and this form holds fewer registers)
          float s4[4];
          masked_scores(s4);
          float tile_max = fmaxf(fmaxf(s4[0], s4[1]), fmaxf(s4[2], s4[3]));
          tile_max = fmaxf(tile_max, shfl_xor_f32(tile_max, 16));
          tile_max = fmaxf(tile_max, shfl_xor_f32(tile_max, 32));
          const float m_new = fmaxf(m[nb], tile_max);
          const float alpha = (m[nb] == m_new) ? 1.f : exp2_hw(m[nb] - m_new);
          m[nb] = m_new;
          dsum[nb] *= alpha;
#pragma unroll
          for (int db = 0; db < 4; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[nb][db][i] *= alpha;
#pragma unroll
          for (int i = 0; i < 4; ++i) pw[i] = exp2_hw(s4[i] - m_new);
        }
        const uint32_t p01 = pack_f16x2(pw[0], pw[1]);
        const uint32_t p23 = pack_f16x2(pw[2], pw[3]);
        dsum[nb] = add_f16x2(p23, add_f16x2(p01, dsum[nb]));
        pb[nb] = __builtin_bit_cast(f16x4, u32x2{p01, p23});
      }

      // stage V (natural layout, swizzled); rows past the last key are zeroed
      // so that no stale or poisoned value can meet a zero weight.
      u32x4 v0, v1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v0[e] = bf16x2_to_f16x2(PF == 1 ? v0r[e] : vc[u][0][e]);
        v1[e] = bf16x2_to_f16x2(PF == 1 ? v1r[e] : vc[u][1][e]);
      }
      if (p * kPageSize + col >= n_k) { v0 = u32x4{}; v1 = u32x4{}; }
      *reinterpret_cast<u32x4*>(stage + page_swizzle(col, 2 * grp)) = v0;
      *reinterpret_cast<u32x4*>(stage + page_swizzle(col, 2 * grp + 1)) = v1;
      if constexpr (PF > 1) {
        advance_ids(p);
        load_page(u, p + PF);
      }
      __asm__ volatile("" ::: "memory");
      // transposed read: lane (grp, j) addresses key 4*grp + j/4, dims 16*db + 4*(j%4)
      const int rkey = 4 * grp + (col >> 2);
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int byte = page_swizzle(rkey, 2 * db + ((col & 3) >> 1)) + 8 * (col & 1);
        const i16x4 vt = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            reinterpret_cast<__attribute__((address_space(3))) i16x4*>(
                reinterpret_cast<uintptr_t>(stage + byte)));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          if (nb < nb_used)
            acc[nb][db] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, vt), pb[nb], acc[nb][db], 0, 0, 0);
      }
      __asm__ volatile("" ::: "memory");
  };
  if constexpr (PF == 1) {
    for (int p = wp0; p < wp1; ++p) page_step(0, p);
  } else {
    int lp = wp0;
    for (; lp + PF <= wp1; lp += PF) {
#pragma unroll
      for (int u = 0; u < PF; ++u) page_step(u, lp + u);
    }
#pragma unroll
    for (int u = 0; u + 1 < PF; ++u)
      if (lp + u < wp1) page_step(u, lp + u);
  }

  // the four lanes of a column hold partial denominators
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    dsum[nb] += shfl_xor_f32(dsum[nb], 16);
    dsum[nb] += shfl_xor_f32(dsum[nb], 32);
  }

  // merge the waves through LDS, one 16-column block at a time
  constexpr int kMB = 1;
  constexpr int kCols = 16 * kMB;
  float* sm_m = reinterpret_cast<float*>(smem);
  float* sm_d = sm_m + NW * kCols;
  float* sm_o = sm_d + NW * kCols;   // [NW][kCols][64 dims]
#pragma unroll
  for (int nb0 = 0; nb0 < NB; nb0 += kMB) {
    if (nb0 >= nb_used) break;                       // uniform
    __syncthreads();                                 // the staging area (or the last round) is free
#pragma unroll
    for (int k = 0; k < kMB; ++k) {
      const int nb = nb0 + k;
      const int jl = 16 * k + col;
      if (grp == 0) {
        sm_m[wave * kCols + jl] = m[nb];
        sm_d[wave * kCols + jl] = dsum[nb];
      }
#pragma unroll
      for (int db = 0; db < 4; ++db)
        *reinterpret_cast<f32x4*>(sm_o + (wave * kCols + jl) * kHeadDim + 16 * db + 4 * grp) = acc[nb][db];
    }
    __syncthreads();

    const int ncols = min(kCols, n_q * G - 16 * nb0);   // real columns of these blocks
    for (int idx = threadIdx.x; idx < ncols * kHeadDim; idx += NW * 64) {
      const int jl = idx / kHeadDim;
      const int d = idx % kHeadDim;
      const int j = 16 * nb0 + jl;
      const int t = j / G;
      const int h = g * G + (j - t * G);
      // each wave's reference is finite (-FLT_MAX until its first visible key)
      float mx = -kFloatMax;
#pragma unroll
      for (int w = 0; w < NW; ++w) mx = fmaxf(mx, sm_m[w * kCols + jl]);
      float den = 0.f, num = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = sm_m[w * kCols + jl];
        const float wt = (mw == mx) ? 1.f : exp2_hw(mw - mx);
        den += wt * sm_d[w * kCols + jl];
        num += wt * sm_o[(w * kCols + jl) * kHeadDim + d];
      }
      const float sink2 = (c == 0 && a.sinks != nullptr) ? a.sinks[h] * kLog2e : kNegInf;
      float lse2;
      // no visible key in the chunk: the key part is empty (d = 0)
      const float o = num * fold_sink(sink2, den > 0.f ? mx : kNegInf, den, &lse2);
      const float lse_nat = lse2 * kLn2;
      const size_t rh = (size_t)(qrow + t) * a.num_qo_heads + h;
      if (S == 1) {
        a.out[rh * kHeadDim + d] = to_bf16_bits(o);
        if (a.lse != nullptr && d == 0) a.lse[rh] = lse_nat;
      } else {
        a.o_part[(rh * S + c) * kHeadDim + d] = o;
        if (d == 0) a.lse_part[rh * S + c] = lse_nat;
      }
    }
  }
}

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
  for (int c = 0; c < N; ++c) {
    if (c >= S) break;
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

}  // namespace

// One-row decode: four waves per workgroup, one page in flight per wave (the
// launch shape measured fastest; deeper rings of pages in flight and eight
// waves per workgroup ran slower).
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const long units = (long)a.batch * a.num_kv_heads * a.num_splits;
  if (units <= 0) return hipSuccess;
  const dim3 grid((unsigned)units), block(4 * 64);
  if (a.max_rows > 0) {   // several query rows per request
    const int cols = a.group * a.max_rows;
    if (a.custom_mask != nullptr) {
      if (cols <= 16) hipLaunchKernelGGL((decode_paged_kernel<4, 1, 1, true, true>), grid, block, 0, stream, a);
      else if (cols <= 32) hipLaunchKernelGGL((decode_paged_kernel<4, 1, 2, true, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((decode_paged_kernel<4, 1, 4, true, true>), grid, block, 0, stream, a);
    } else {
      if (cols <= 16) hipLaunchKernelGGL((decode_paged_kernel<4, 1, 1, true, false>), grid, block, 0, stream, a);
      else if (cols <= 32) hipLaunchKernelGGL((decode_paged_kernel<4, 1, 2, true, false>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((decode_paged_kernel<4, 1, 4, true, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError();
  }
  hipLaunchKernelGGL((decode_paged_kernel<4, 1, 1, false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  const long n = (long)a.rows * a.num_heads;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(merge_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sinkattn
