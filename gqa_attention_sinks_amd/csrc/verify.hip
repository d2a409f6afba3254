// Verify decode with per-head attention sinks: several query rows per request
// over a paged cache (the verify step of speculative decoding), with an
// optional bit-packed custom mask per request (a draft tree).
//
// Method: Perplexity blog "GPT-OSS on day 0" (French rendering "GPT-OSS au
// jour J"), section "Kernels for GPT-OSS > Sink attention": the streaming
// softmax keeps a running max m and a scale d seeded with the head's sink, and
// when the KV sequence is split into blocks only the first block carries the
// sink.  Verify step, draft trees and CPU-built page metadata: "Accelerating
// Sonar through speculation", sections "Speculative decoding" and "Inference
// with speculative decoding".
//
// Work decomposition (gfx950, 64-lane waves):
//   workgroup = (request b, KV head g, chunk c), four waves: the chunk's pages
//   are split into four contiguous runs, one per wave, and the waves merge
//   through LDS at the end.  The MFMA columns are the request's (row, head)
//   pairs, column j = (row j / G, head j % G), at most 64, in two 32-column
//   blocks (the second one skipped, wave-uniformly, when the request has at
//   most 32 columns).  Per step of two pages (32 keys) and column block:
//     S^T[32 keys x 32 cols] = K . Q^T        -> 4 x MFMA 32x32x16 bf16
//       K is read in contiguous rows, staged per wave in LDS and read back in
//       the A operand layout (lane l: key l % 32, dims 16 ks + 8 (l / 32)
//       .. + 7); the Q^T operands are staged in LDS once
//     weights exp2(s c - m) against a reference per column that moves only
//     when some weight would pass 2^14 (then: the column maxima, a rescale
//     and the weights again), summed from the same fp16 values that feed P.V
//     O^T[64 dims x 32 cols] += V^T . P^T    -> 4 x MFMA 32x32x16 fp16
//       V converted to fp16 and staged per wave in LDS as [key][dim], read
//       back transposed with ds_read_b64_tr_b16; P^T is the score
//       accumulator converted to fp16
//   so one softmax instruction chain covers 32 columns x 32 keys (a lane: 16
//   keys of one column).  The next step's pages are in flight while a step
//   computes.  The sink is folded in once the waves have merged (fold_sink),
//   which gives exactly the state of the sink-seeded recurrence.

#include "decode_common.hpp"
#include "device_common.hpp"
#include "kernel_args.hpp"
#include "mfma_tile.hpp"

namespace sinkattn {
namespace {

constexpr int kVW = 4;                                  // waves per workgroup
constexpr int kVThreads = kVW * 64;
constexpr int kStepKeys = 2 * kPageSize;                // keys per step: two pages
constexpr int kStageBytes = kStepKeys * kHeadDim * 2;   // a wave's V of one step, fp16: 4 KiB
constexpr float kSumLimit = 16384.f;                    // 2^14
constexpr int kMaxRows = 8;                             // query rows per request at most
constexpr float kFloatMax = 3.402823466e38f;
// s_waitcnt operand: vector memory count 0, the other counters unconstrained
// (vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVm0 = 0x0F70;

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// LDS of a workgroup: the waves' V stages and the Q^T operands while pages
// are processed; the merge of one column block after the page loop (waves
// 1..3 leave their state, wave 0 combines it with its own).
struct VerifySmem {
  union {
    struct {
      uint8_t stage[kVW][kStageBytes];    // V of the wave's step, fp16
      uint8_t kstage[kVW][kStageBytes];   // K of the wave's step, bf16
      u32x4 q[2][4][64];                 // [column block][k step][lane]
    } run;
    struct {
      float o[kVW - 1][2][16][64];       // [wave - 1][dim block][accumulator element][lane]
      float m[kVW - 1][32];
      float d[kVW - 1][32];
    } merge;
  } u;
};

// Four mask bits of keys key0 .. key0 + 3 for the row whose bits start at
// bit `row_bit` of the request's mask; keys at or past n_k read as hidden,
// and no byte past the row's last key is read.
__device__ __forceinline__ uint32_t mask4(const uint8_t* mbytes, int row_bit, int key0, int n_k) {
  if (key0 >= n_k) return 0u;
  const int bit0 = row_bit + key0;
  const int bit1 = row_bit + min(key0 + 3, n_k - 1);
  uint32_t w = mbytes[bit0 >> 3];
  if ((bit1 >> 3) != (bit0 >> 3)) w |= (uint32_t)mbytes[bit1 >> 3] << 8;
  const int valid = min(4, n_k - key0);
  return (w >> (bit0 & 7)) & ((1u << valid) - 1u);
}

template <bool MASK>
__global__ __launch_bounds__(kVThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void verify_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) VerifySmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: bookkeeping stays scalar
  const int r32 = lane & 31;   // MFMA column within a 32-column block / key within a step
  const int half = lane >> 5;  // which 8-element k slice / 4-key group this lane holds
  const int S = a.num_splits;
  const int G = a.group;

  const DecodeUnit du = decode_unit<kVW>(a);
  const int b = __builtin_amdgcn_readfirstlane(du.b);
  const int g = du.g, c = du.c;
  const int r0 = a.qo_indptr[b];
  const int qrow = __builtin_amdgcn_readfirstlane(r0);
  const int n_q = __builtin_amdgcn_readfirstlane(min(a.qo_indptr[b + 1] - r0, a.max_rows));
  if (n_q < 1) return;                                   // uniform: an empty request
  const int nb_used = (n_q * G + 31) / 32;               // column blocks the request fills

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
  const int per_wave = (pg1 - pg0 + kVW - 1) / kVW;
  const int wp0 = min(pg0 + wave * per_wave, pg1);
  const int wp1 = min(wp0 + per_wave, pg1);
  const int run_end = min(wp1 * kPageSize, t_hi);        // this wave's keys: [wp0 * 16, run_end)
  // keys every row of the request sees: [full_lo, full_hi] within the chunk
  const int full_lo = a.window > 0 ? max(t_lo, n_k - a.window) : t_lo;
  const int full_hi = min(t_hi - 1, n_k - n_q);

  const int32_t* pages = a.page_indices + __builtin_amdgcn_readfirstlane(du.page_base);
  const size_t head_stride = (size_t)kPageSize * kHeadDim;          // elements per (page, KV head)
  const size_t page_stride = (size_t)a.num_kv_heads * head_stride;  // elements per page
  const uint16_t* kpool = a.k_pool + (size_t)g * head_stride;
  const uint16_t* vpool = a.v_pool + (size_t)g * head_stride;
  // K and V are read in contiguous kilobytes, 16 bytes a lane: load j holds
  // key 8 j + lane / 8 of the step (page a for j < 2, else page b), chunk
  // lane % 8; both go through LDS (whole runs per load stream faster than the
  // operand layout's 16-byte pieces: 65.8 against 59.1 us for the loads alone
  // on the verify batch)
  const int v_key = lane >> 3, v_chunk = lane & 7;
  uint8_t* stage = sm.u.run.stage[wave];
  uint8_t* kstage = sm.u.run.kstage[wave];
  const uint32_t kstage0 = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)kstage;
  const uint32_t stage0 = (uint32_t)(size_t)(__attribute__((address_space(3))) uint8_t*)stage;
  const TileLanes tl = tile_lanes(lane);

  // Page ids of the wave's run arrive as vector loads, one lane per page, in
  // two registers of 64 (even and odd groups); entering group g reloads the
  // register of group g - 1 with group g + 1, 64 pages ahead of its use.
  // They go out first: the first pages wait for them.
  int ids0 = lane < wp1 - wp0 ? pages[wp0 + lane] : 0;
  int ids1 = 64 + lane < wp1 - wp0 ? pages[wp0 + 64 + lane] : 0;

  // Q^T operands: entry [cb][ks][l] holds column 32 cb + l % 32, dims
  // 16 ks + 8 (l / 32) .. + 7 (zero for columns past the request's rows)
  for (int e = tid; e < 2 * 4 * 64; e += kVThreads) {
    const int l = e & 63, ks = (e >> 6) & 3, cb = e >> 8;
    const int j = 32 * cb + (l & 31);
    const int t = j / G;
    u32x4 x = {};
    if (t < n_q)
      x = ldg16(a.q + ((size_t)(qrow + t) * a.num_qo_heads + g * G + (j - t * G)) * kHeadDim + 16 * ks +
                8 * (l >> 5));
    sm.u.run.q[cb][ks][l] = x;
  }
  // this lane's column of each block and the keys of the chunk it may see
  int v_lo[2], v_hi[2], c_bit[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int t = (32 * cb + r32) / G;
    const int c_pos = n_k - n_q + t;
    const int c_lo = a.window > 0 ? c_pos - a.window + 1 : 0;
    v_lo[cb] = MASK ? t_lo : max(t_lo, c_lo);
    v_hi[cb] = t < n_q ? (MASK ? t_hi - 1 : min(t_hi - 1, c_pos)) : -1;   // a column past the rows sees nothing
    c_bit[cb] = t < n_q ? t * n_k : -1;
  }
  int next_group = 1;
  auto page_id = [&](int p) -> int {      // p uniform, in the current group or the next
    const int r = p - wp0;
    return ((r >> 6) & 1) ? __builtin_amdgcn_readlane(ids1, r & 63) : __builtin_amdgcn_readlane(ids0, r & 63);
  };
  auto advance_ids = [&](int p) {         // p: the first page of the step being processed
    const int gr = (p - wp0) >> 6;
    if (gr == next_group) {
      ++next_group;
      const int base = wp0 + 64 * (gr + 1);
      if (gr & 1) ids0 = base + lane < wp1 ? pages[base + lane] : 0;
      else ids1 = base + lane < wp1 ? pages[base + lane] : 0;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
  };
  // The step at page p: K and V of pages p and p + 1 (past the run the last
  // page again) in contiguous rows.  Two
  // register sets alternate between steps: each step first loads the next
  // step's pages into the set the previous step has finished with, so they
  // are in flight while it computes (a third set, two steps ahead, measured
  // slower: more pages in flight cost more than the latency they hide).
  // Every path issues the same loads (a step past the run reloads the run's
  // last pages, a cache hit): the compiler's count of loads in flight then
  // stays exact, and a step waits for its own pages only.
  const int n_steps = (wp1 - wp0 + 1) / 2;
  const int p_last = wp0 + 2 * max(n_steps - 1, 0);    // the run's last step
  u32x4 kA[4], vA[4], kB[4], vB[4];
  auto load_step = [&](int p, u32x4 (&kc)[4], u32x4 (&vc)[4]) {
    p = min(p, p_last);
    const int id_a = page_id(p);
    const int id_b = page_id(min(p + 1, wp1 - 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t off = (size_t)(j < 2 ? id_a : id_b) * page_stride + (j & 1) * 8 * kHeadDim + 8 * lane;
      kc[j] = ldg16(kpool + off);
      vc[j] = ldg16(vpool + off);
    }
  };

  // the ids (and Q) have arrived: the first step's pages go out now, so
  // that they are in flight during the mask scan
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  if (n_steps > 0) load_step(wp0, kA, vA);
  const uint8_t* mbytes = MASK ? a.custom_mask + a.mask_indptr[b] : nullptr;
  // MASK: per row, the first hidden key of the chunk (t_hi when none).  The
  // steps below it show all their keys to that row, so only the others read
  // mask bits per lane; a draft tree shows its rows the whole context, so that
  // is every step but the last one or two.  One pass over the chunk's bits,
  // 32 keys per thread and word (the bytes read stop at the row's last key).
  __shared__ int s_fz[kMaxRows];
  int fz[2] = {0x7fffffff, 0x7fffffff};
  if (MASK) {
    if (tid < kMaxRows) s_fz[tid] = t_hi;
    __syncthreads();
    const int nw = t_hi > t_lo ? (t_hi - t_lo + 31) / 32 : 0;   // words per row
    for (int w = tid; w < n_q * nw; w += kVThreads) {
      const int t = w / nw;
      const int key0 = t_lo + 32 * (w - t * nw);
      const int n = min(32, t_hi - key0);
      const int bit0 = t * n_k + key0;
      const int last = (bit0 + n - 1) >> 3;
      uint64_t x = 0;
#pragma unroll
      for (int i = 0; i < 5; ++i) x |= (uint64_t)mbytes[min((bit0 >> 3) + i, last)] << (8 * i);
      const uint32_t valid = n == 32 ? 0xFFFFFFFFu : ((1u << n) - 1u);
      const uint32_t hidden = ~(uint32_t)(x >> (bit0 & 7)) & valid;
      if (hidden != 0u) atomicMin(&s_fz[t], key0 + __builtin_ctz(hidden));
    }
  }
  __syncthreads();
  if (MASK) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const int t = (32 * cb + r32) / G;
      if (t < n_q) fz[cb] = s_fz[t];
    }
  }

  // Key-domain state per column block: reference m (base 2; at or below the
  // key maximum seen), this lane's part of the denominator, O^T accumulator.
  float m[2] = {-kFloatMax, -kFloatMax}, dsum[2] = {0.f, 0.f};
  f32x16 acc[2][2] = {};   // [column block][dim block]
  const float cs = a.scale_log2;

  // step st with its pages in (kc, vc); (kn, vn): the other set
  auto step = [&](const int st, u32x4 (&kc)[4], u32x4 (&vc)[4], u32x4 (&kn)[4], u32x4 (&vn)[4])
      __attribute__((always_inline)) {
    const int p = wp0 + 2 * st;
    const int key_base = p * kPageSize;
    // the next step's pages, into the set the previous step has finished with
    advance_ids(min(p + 2, p_last));
    load_step(p + 2, kn, vn);
    // K of the step through the wave's LDS stage: rows in, operand layout out
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<u32x4*>(kstage + tile_swizzle(8 * j + v_key, v_chunk)) = kc[j];
    __asm__ volatile("" ::: "memory");
    bf16x8 kop[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kop[ks] = *lds_at<const bf16x8>(kstage0 + tl.k[ks]);
    // scores of the step, every column block the request fills
    f32x16 s[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      s[cb] = f32x16{};
      if (cb >= nb_used) continue;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        s[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks],
                                                        __builtin_bit_cast(bf16x8, sm.u.run.q[cb][ks][lane]),
                                                        s[cb], 0, 0, 0);
    }
    // V of the step as fp16 into the wave's stage; rows past the wave's keys
    // are zeroed so that no stale or poisoned value meets a zero weight
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool key_ok = key_base + 8 * j + v_key < run_end;
      u32x4 v16;
#pragma unroll
      for (int e = 0; e < 4; ++e) v16[e] = key_ok ? bf16x2_to_f16x2(vc[j][e]) : 0u;
      *reinterpret_cast<u32x4*>(stage + tile_swizzle(8 * j + v_key, v_chunk)) = v16;
    }
    __asm__ volatile("" ::: "memory");

    // visibility: the common step shows every key to every real column
    const bool step_in = key_base >= t_lo && key_base + kStepKeys <= run_end;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      if (cb >= nb_used) continue;
      bool full;
      if (MASK) full = step_in && __builtin_amdgcn_ballot_w64(c_bit[cb] >= 0 && key_base + kStepKeys > fz[cb]) == 0;
      else full = step_in && key_base >= full_lo && key_base + kStepKeys - 1 <= full_hi;
      if (!full) {   // uniform: the chunk's edges, the diagonal, the window edge, masks with holes
        uint32_t mb = 0xFFFFu;   // MASK: bit i = element i of the lane's scores
        if (MASK) {
          mb = 0u;
          if (c_bit[cb] >= 0) {
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) mb |= mask4(mbytes, c_bit[cb], key_base + 8 * q4 + 4 * half, n_k) << (4 * q4);
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key_base + 8 * (i >> 2) + 4 * half + (i & 3);
          bool vis = key >= v_lo[cb] && key <= v_hi[cb] && key < run_end;
          if (MASK) vis = vis && ((mb >> i) & 1u);
          s[cb][i] = vis ? s[cb][i] : kNegInf;
        }
      }
    }

    // fp16 weights against the reference; a column whose weight share would
    // pass 2^14 (always on its first visible keys) moves the reference up
    f16x8 pop[2][2];
    float tsum[2] = {0.f, 0.f};
    auto weights = [&](int cb) {
      f16x2 h[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float lo = exp2_hw(__builtin_fmaf(s[cb][2 * j], cs, -m[cb]));
        const float hi = exp2_hw(__builtin_fmaf(s[cb][2 * j + 1], cs, -m[cb]));
        h[j] = __builtin_bit_cast(f16x2, pack_f16x2(lo, hi));
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        pop[cb][hh] = __builtin_bit_cast(f16x8, u32x4{__builtin_bit_cast(uint32_t, h[4 * hh]),
                                                      __builtin_bit_cast(uint32_t, h[4 * hh + 1]),
                                                      __builtin_bit_cast(uint32_t, h[4 * hh + 2]),
                                                      __builtin_bit_cast(uint32_t, h[4 * hh + 3])});
      const f16x2 t = ((h[0] + h[1]) + (h[2] + h[3])) + ((h[4] + h[5]) + (h[6] + h[7]));
      tsum[cb] = (float)t[0] + (float)t[1];
    };
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      if (cb < nb_used) weights(cb);
    if (__builtin_amdgcn_ballot_w64(tsum[0] > kSumLimit || tsum[1] > kSumLimit) != 0) {
      __asm__ volatile("");
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        if (cb >= nb_used) continue;
        float mx = s[cb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[cb][i]);
        mx = fmaxf(mx, shfl_xor_f32(mx, 32));
        // a column with no visible key here keeps its reference (mx = -inf)
        const float m_new = fmaxf(m[cb], mx * cs);
        const float alpha = exp2_hw(m[cb] - m_new);
        m[cb] = m_new;
        dsum[cb] *= alpha;
#pragma unroll
        for (int db = 0; db < 2; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[cb][db][i] *= alpha;
        weights(cb);
      }
    }
    dsum[0] += tsum[0];
    dsum[1] += tsum[1];

    // O^T += V^T . P^T: the transposed V operands of the step's two 16-key
    // halves and both dim blocks (keys in the order of the score elements)
    f16x8 vt[2][2];   // [16-key half][dim block]
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_at<i16x4>(stage0 + tl.v[db][0] + hh * 16 * 128));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_at<i16x4>(stage0 + tl.v[db][1] + hh * 16 * 128));
        typedef __attribute__((ext_vector_type(8))) short i16x8;
        vt[hh][db] = __builtin_bit_cast(f16x8, i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      if (cb >= nb_used) continue;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int db = 0; db < 2; ++db)
          acc[cb][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vt[hh][db], pop[cb][hh], acc[cb][db], 0, 0, 0);
    }
    __asm__ volatile("" ::: "memory");
  };
  int st = 0;
  for (; st + 1 < n_steps; st += 2) {
    step(st, kA, vA, kB, vB);
    step(st + 1, kB, vB, kA, vA);
  }
  if (st < n_steps) step(st, kA, vA, kB, vB);

  // the two lanes of a column hold the denominator shares of different keys
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) dsum[cb] += shfl_xor_f32(dsum[cb], 32);

  // merge the waves through LDS, one column block at a time: waves 1..3 leave
  // their state, wave 0 combines it with its own and writes the result
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    if (cb >= nb_used) break;                            // uniform
    __syncthreads();                                     // stages, Q and the last round are free
    if (wave > 0) {
      if (half == 0) {
        sm.u.merge.m[wave - 1][r32] = m[cb];
        sm.u.merge.d[wave - 1][r32] = dsum[cb];
      }
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.u.merge.o[wave - 1][db][i][lane] = acc[cb][db][i];
    }
    __syncthreads();
    const int j = 32 * cb + r32;
    const int t = j / G;
    if (wave == 0 && t < n_q) {
      const int h = g * G + (j - t * G);
      // each wave's reference is finite (-FLT_MAX until its first visible key)
      float mx = m[cb];
#pragma unroll
      for (int w = 0; w < kVW - 1; ++w) mx = fmaxf(mx, sm.u.merge.m[w][r32]);
      float wt[kVW];
      wt[0] = (m[cb] == mx) ? 1.f : exp2_hw(m[cb] - mx);
      float den = wt[0] * dsum[cb];
#pragma unroll
      for (int w = 0; w < kVW - 1; ++w) {
        const float mw = sm.u.merge.m[w][r32];
        wt[w + 1] = (mw == mx) ? 1.f : exp2_hw(mw - mx);
        den += wt[w + 1] * sm.u.merge.d[w][r32];
      }
      const float sink2 = (c == 0 && a.sinks != nullptr) ? a.sinks[h] * kLog2e : kNegInf;
      float lse2;
      // no visible key in the chunk: the key part is empty (d = 0)
      const float inv = fold_sink(sink2, den > 0.f ? mx : kNegInf, den, &lse2);
      const float lse_nat = lse2 * kLn2;
      const size_t rh = (size_t)(qrow + t) * a.num_qo_heads + h;
#pragma unroll
      for (int db = 0; db < 2; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * q4 + e;
            float num = wt[0] * acc[cb][db][i];
#pragma unroll
            for (int w = 0; w < kVW - 1; ++w) num += wt[w + 1] * sm.u.merge.o[w][db][i][lane];
            o[e] = num * inv;
          }
          const int d0 = 32 * db + 8 * q4 + 4 * half;
          if (S == 1) {
            u32x2 x;
            x[0] = pack_bf16x2(o[0], o[1]);
            x[1] = pack_bf16x2(o[2], o[3]);
            *reinterpret_cast<u32x2*>(a.out + rh * kHeadDim + d0) = x;
          } else {
            *reinterpret_cast<f32x4*>(a.o_part + (rh * S + c) * kHeadDim + d0) = f32x4{o[0], o[1], o[2], o[3]};
          }
        }
      if (half == 0) {
        if (S == 1) {
          if (a.lse != nullptr) a.lse[rh] = lse_nat;
        } else {
          a.lse_part[rh * S + c] = lse_nat;
        }
      }
    }
  }
}

}  // namespace

// Several query rows per request: one workgroup per (request, KV head, chunk).
hipError_t launch_decode_verify(const DecodeArgs& a, hipStream_t stream) {
  const long units = (long)a.batch * a.num_kv_heads * a.num_splits;
  if (units <= 0) return hipSuccess;
  const dim3 grid((unsigned)units), block(kVThreads);
  if (a.custom_mask != nullptr) hipLaunchKernelGGL(verify_kernel<true>, grid, block, 0, stream, a);
  else hipLaunchKernelGGL(verify_kernel<false>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace sinkattn
