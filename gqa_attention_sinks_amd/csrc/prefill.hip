// Causal / sliding-window prefill with per-head attention sinks.
//
// Method: Perplexity blog "GPT-OSS on day 0" (French rendering "GPT-OSS au
// jour J"), section "Kernels for GPT-OSS > Sink attention": the sink is one
// more term of the softmax; the streaming softmax (running max m, scale d)
// starts from (sink, 1), so the sink costs nothing per key.
//
// Work decomposition (gfx950):
//   workgroup = 4 waves of 64 query rows each (two 32-row MFMA blocks, so
//   every K/V operand read from LDS feeds two MFMAs): the same 64 rows of four
//   query heads that share a KV head when the GQA group splits into fours
//   (every wave then needs exactly the workgroup's key tiles), else 256
//   consecutive rows of one head.  Two workgroups per CU, so each SIMD runs
//   two waves (one of each); inside a wave the matrix steps are interleaved
//   with the vector work of the other half tile.  Consecutive workgroup
//   ids walk the KV heads first, so with 8 KV heads and 8 XCDs each XCD's L2
//   serves one KV head.  Tiles of a request are issued longest first (causal
//   work grows with the row index).
//   Per KV tile of 64 keys (K and V staged in LDS, double buffered, 16-byte
//   chunks swizzled so that every LDS access pattern below is free of bank
//   conflicts):
//     S^T[64 keys x 64 rows] = K . Q^T    -> 16 x MFMA 32x32x16 bf16 (Q^T in registers)
//     base-2 online softmax on the accumulator: each lane holds two query
//     rows and 32 of their keys
//     O^T[64 dims x 64 rows] += V^T . P^T -> 16 x MFMA 32x32x16 fp16
//       (P^T is the score accumulator converted to fp16; V is converted to
//        fp16 once when its tile is staged, and V^T comes from the natural
//        [key][dim] LDS tile through ds_read_b64_tr_b16).  fp16 weights carry
//        three more mantissa bits than bf16; they are taken relative to a
//        reference at or below the running key maximum, and the sink is
//        folded in at the end, which gives exactly the state of the
//        sink-seeded recurrence.
//   The reference moves only when it must: a tile's weights are first taken
//   against the current reference, and only if some lane's share of a row's
//   weight sum exceeds 2^14 (a key far above the reference; fp16 weights stay
//   finite below 65504) does the wave find the tile's row maxima, move the
//   reference up, rescale and recompute.  A workgroup's first key tile
//   instead takes the reference from the row maxima of its first half
//   before any weight (it starts at -FLT_MAX); later tiles almost never
//   move it.
//   Masking is applied only on tiles that cross the causal diagonal or the
//   window's lower edge.

#include <type_traits>

#include "device_common.hpp"
#include "kernel_args.hpp"
#include "mfma_tile.hpp"

namespace sinkattn {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 64;               // two 32-row MFMA blocks per wave
constexpr int kBN = kPrefillTileKeys;          // keys per tile
constexpr int kTileBytes = kBN * kHeadDim * 2;   // 8 KiB
constexpr float kSumLimit = 16384.f;           // 2^14
constexpr float kFloatMax = 3.402823466e38f;

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds_ptr(uint8_t* p) {
  return (__attribute__((address_space(3))) T*)(p);
}

// A per-tile LDS base (stage address + lane offset) that the compiler may not
// re-associate with the constant part of each read: otherwise it hoists one
// precomputed address per read out of the loop (a register and two adds each).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  __asm__ volatile("" : "+v"(x));
  return x;
}

// Scheduling hints: issue a block's `reads` LDS reads before its first MFMA,
// so that their latencies overlap instead of each read waiting for the MFMAs
// before it (which is what the register-pressure-driven default does).
template <int READS, int MFMAS>
__device__ __forceinline__ void reads_then_mfmas() {
  __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
  __builtin_amdgcn_sched_group_barrier(0x008, MFMAS, 0);
}

// Key tiles a query tile of RT rows spans (the work of a workgroup, in
// 64-key tiles).
template <int RT>
__device__ __forceinline__ int tile_work(int n_q, int n_k, int t, int window) {
  const int shift = n_k - n_q;
  const int t0 = t * RT;
  const int t_last = min(t0 + RT, n_q) - 1;
  const int lo_first = window > 0 ? max(0, shift + t0 - window + 1) : 0;
  const int k_first = (lo_first / kBN) * kBN;
  return (shift + t_last + 1 - k_first + kBN - 1) / kBN;
}

static_assert(kPrefillRankMaxTiles == kWaves * 64, "ranking lists one tile per thread");

// Find the (request, tile) handled by tile slot `slot`.  Tiles are numbered
// request by request (every thread sums a run of requests, then a block
// scan).  When the requests differ in shape, the batch has at most 256
// query tiles and the window is unbounded or longer than kPlanMinWindow, the
// slots take the tiles in order of decreasing work (ties by number), so the
// longest tiles of every request start first and the short ones fill the
// tail.  Otherwise they take them request by request, longest
// tile first: with equal requests that order is as balanced, tiles of one
// request that run together share its keys in L2, and under a short window
// every tile carries about the same work (a few key tiles), so ranking would
// only cost time.
template <int RT>
__device__ bool locate_tile(const PrefillArgs& a, int slot, int* s_scan, int* out_b, int* out_tile) {
  constexpr int kThreads = kWaves * 64;
  const int tid = threadIdx.x;
  const int per = (a.batch + kThreads - 1) / kThreads;
  const int b0 = min(tid * per, a.batch);
  const int b1 = min(b0 + per, a.batch);
  auto req_tiles = [&](int b) {
    const int n = a.qo_indptr[b + 1] - a.qo_indptr[b];
    return (a.skip_single_rows && n == 1) ? 0 : (n + RT - 1) / RT;
  };
  auto req_len = [&](int b, int* n_q, int* n_k) {
    *n_q = a.qo_indptr[b + 1] - a.qo_indptr[b];
    *n_k = a.paged ? a.kv_len[b] : a.kv_indptr[b + 1] - a.kv_indptr[b];
  };
  int local = 0;
  bool same_shape = true;   // every request shaped like request 0
  int q0, k0;
  req_len(0, &q0, &k0);
  for (int b = b0; b < b1; ++b) {
    local += req_tiles(b);
    int nq, nk;
    req_len(b, &nq, &nk);
    same_shape = same_shape && nq == q0 && nk == k0;
  }
  const bool uniform = __syncthreads_and(same_shape);
  s_scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {
    const int v = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  const int excl = s_scan[tid] - local;
  const int total = s_scan[kThreads - 1];
  __shared__ int s_found[2];
  if (tid == 0) s_found[0] = -1;
  if (total <= kThreads && !uniform && (a.window == 0 || a.window > kPlanMinWindow)) {
    // list every (request, tile) with its work, then rank
    __shared__ int s_work[kThreads];
    __shared__ int s_req[kThreads];
    __shared__ int s_tile[kThreads];
    int pos = excl;
    for (int b = b0; b < b1; ++b) {
      const int nt = req_tiles(b);
      if (nt == 0) continue;
      int n_q, n_k;
      req_len(b, &n_q, &n_k);
      for (int t = 0; t < nt; ++t, ++pos) {
        s_work[pos] = tile_work<RT>(n_q, n_k, t, a.window);
        s_req[pos] = b;
        s_tile[pos] = t;
      }
    }
    __syncthreads();
    if (tid < total) {
      const int w = s_work[tid];
      int rank = 0;
      for (int q = 0; q < total; ++q) {
        const int wq = s_work[q];
        rank += (wq > w) || (wq == w && q < tid);
      }
      if (rank == slot) {   // ranks are a permutation: at most one writer
        s_found[0] = s_req[tid];
        s_found[1] = s_tile[tid];
      }
    }
    __syncthreads();
  } else {
    __syncthreads();
    if (slot >= excl && slot < excl + local) {
      int base = excl;
      for (int b = b0; b < b1; ++b) {
        const int nt = req_tiles(b);
        if (slot < base + nt) {
          s_found[0] = b;
          s_found[1] = nt - 1 - (slot - base);   // longest tile first
          break;
        }
        base += nt;
      }
    }
    __syncthreads();
  }
  *out_b = s_found[0];
  *out_tile = s_found[1];
  return s_found[0] >= 0;
}

// The second kernel argument: the host plan, or a placeholder for launches
// whose workgroups find their tile themselves.
template <bool PLANNED> struct PlanArg { uint32_t unused; };
template <> struct PlanArg<true> { PrefillPlan p; };

// HP: query heads per workgroup.  HP = 1: the four waves take four 64-row
// blocks of one head (256 rows a tile).  HP = 4: they take the same 64 rows
// of four heads that share a KV head, so every wave needs exactly the
// workgroup's key tiles (no wave waits out another's diagonal or window
// edge).  PLANNED: each slot's (request, tile) comes from the host plan.
template <bool PAGED, int HP, bool PLANNED>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillArgs a, PlanArg<PLANNED> plan) {
  constexpr int RT = kRowsPerWave * (kWaves / HP);   // query rows of a workgroup tile
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * 2 * kTileBytes];
  __shared__ int s_scan[kWaves * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: bookkeeping stays scalar
  const int r32 = lane & 31;    // MFMA column: query row within a 32-row block
  const int half = lane >> 5;   // which 8-element k-slice / 4-key group this lane holds

  int id = blockIdx.x;
  const int g = id % a.num_kv_heads;
  id /= a.num_kv_heads;
  const int hgroups = a.group / HP;                 // head groups of one KV head
  const int hg = id % hgroups;
  const int slot = id / hgroups;
  const int head = g * a.group + hg * HP + (HP > 1 ? wave : 0);   // this wave's query head

  int b, tile;
  if constexpr (PLANNED) {   // every slot of a planned launch holds a tile
    const uint32_t e = plan.p.slot[slot];
    b = (int)(e >> 16);
    tile = (int)(e & 0xffffu);
  } else {
    if (!locate_tile<RT>(a, slot, s_scan, &b, &tile)) return;   // uniform over the workgroup
    b = __builtin_amdgcn_readfirstlane(b);
    tile = __builtin_amdgcn_readfirstlane(tile);
  }

  const int q_begin = a.qo_indptr[b];
  const int n_q = a.qo_indptr[b + 1] - q_begin;
  int n_k, kv_begin = 0;
  if (PAGED) {
    n_k = a.kv_len[b];
  } else {
    kv_begin = a.kv_indptr[b];
    n_k = a.kv_indptr[b + 1] - kv_begin;
  }
  const int shift = n_k - n_q;   // row t sits at key position shift + t
  const int t0 = tile * RT;
  const int t_last = min(t0 + RT, n_q) - 1;
  const int W = a.window;
  const int lo_first = W > 0 ? max(0, shift + t0 - W + 1) : 0;
  const int k_first = (lo_first / kBN) * kBN;
  const int k_end = shift + t_last + 1;   // exclusive
  const int ntiles = (k_end - k_first + kBN - 1) / kBN;

  // this wave's 64 rows (two 32-row MFMA blocks) and the two rows of this lane
  const int wt0 = t0 + (HP > 1 ? 0 : kRowsPerWave * wave);
  const bool wave_live = wt0 <= t_last;
  const int wp_min = shift + wt0;
  const int wp_max = shift + min(wt0 + kRowsPerWave - 1, t_last);
  int my_t[2], my_p[2], my_lo[2];
  bf16x8 qop[2][4];   // Q^T operands: column = row, k = dims 16*ks + 8*half + e
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    my_t[rb] = wt0 + 32 * rb + r32;
    my_p[rb] = shift + my_t[rb];
    my_lo[rb] = W > 0 ? my_p[rb] - W + 1 : 0;
    const bool ok = my_t[rb] < n_q;
    const uint16_t* qp = a.q + ((size_t)(q_begin + (ok ? my_t[rb] : 0)) * a.num_qo_heads + head) * kHeadDim + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qop[rb][ks] = ok ? __builtin_bit_cast(bf16x8, ldg16(qp + 16 * ks)) : bf16x8{};
  }

  // Key-domain streaming state per row: reference m (base 2; at or below the
  // key maximum seen), this lane's part of the denominator, and the P.V
  // accumulator.  The sink is folded in at the end (fold_sink), which yields
  // the state of the sink-seeded recurrence.
  float m[2] = {-kFloatMax, -kFloatMax}, dsum[2] = {0.f, 0.f};
  // the head's sink, loaded now so that its latency is not paid at the end
  const float sink2 = a.sinks != nullptr ? a.sinks[head] * kLog2e : kNegInf;
  f32x16 acc[2][2] = {};   // [row block][dim block]
  const float c = a.scale_log2;
  const TileLanes tl = tile_lanes(lane);
  const uint32_t smem0 = (uint32_t)(size_t)lds_ptr<uint8_t>(smem);   // LDS byte address

  // Staging: a wave stages sixteen consecutive keys (they share a page), each
  // load a contiguous kilobyte of rows: lane -> keys lane/8 and 8 + lane/8,
  // 16 bytes at chunk lane%8 of K and of V.  The address is a uniform base
  // (scalar registers) plus a fixed per-lane offset.  Keys past the last one
  // re-read the last key and are zeroed when staged, so the common full tile
  // carries no per-row checks.
  const int wkey = 16 * wave;       // first key of this wave's rows
  const int lkey = lane >> 3;       // this lane's first key among them (the second: lkey + 8)
  const int ld_c = lane & 7;        // this lane's 16-byte chunk
  const int32_t* page_list = PAGED ? a.page_indices + a.kv_indptr[b] : nullptr;
  const uint32_t key_bytes = PAGED ? kHeadDim * 2 : (uint32_t)a.num_kv_heads * kHeadDim * 2;
  const uint32_t lane_off_full = (uint32_t)lkey * key_bytes + ld_c * 16;
  const uint32_t half_off = 8 * key_bytes;   // keys 8..15 of the wave
  const uint8_t* kbytes = reinterpret_cast<const uint8_t*>(a.k);
  const uint8_t* vbytes = reinterpret_cast<const uint8_t*>(a.v);
  // paged: the page holding the wave's first (clamped) key, fetched a tile ahead
  auto page_of = [&](int kt) -> int {
    return page_list[min(kt + wkey, n_k - 1) / kPageSize];
  };
  auto load_tile = [&](int kt, int page, u32x4 (&kr)[2], u32x4 (&vr)[2]) {
    const int k0 = min(kt + wkey, n_k - 1);
    const size_t base = PAGED ? ((size_t)page * a.num_kv_heads + g) * (kPageSize * kHeadDim * 2)
                              : ((size_t)(kv_begin + k0) * a.num_kv_heads + g) * (kHeadDim * 2);
    uint32_t off0 = lane_off_full, off1 = lane_off_full + half_off;
    if (kt + kBN > n_k) {            // uniform: only the range's last tile
      __asm__ volatile("");
      const int key0 = min(kt + wkey + lkey, n_k - 1);
      const int key1 = min(kt + wkey + 8 + lkey, n_k - 1);
      off0 = (uint32_t)(PAGED ? key0 % kPageSize : key0 - k0) * key_bytes + ld_c * 16;
      off1 = (uint32_t)(PAGED ? key1 % kPageSize : key1 - k0) * key_bytes + ld_c * 16;
    }
    kr[0] = *reinterpret_cast<const u32x4*>(kbytes + base + off0);
    kr[1] = *reinterpret_cast<const u32x4*>(kbytes + base + off1);
    vr[0] = *reinterpret_cast<const u32x4*>(vbytes + base + off0);
    vr[1] = *reinterpret_cast<const u32x4*>(vbytes + base + off1);
  };
  // Rows past the last key are staged as zeros.
  auto fix_tail = [&](int kt, u32x4 (&kr)[2], u32x4 (&vr)[2]) {
    if (kt + kBN > n_k) {            // uniform: only the range's last tile
      __asm__ volatile("");
      if (kt + wkey + lkey >= n_k) kr[0] = vr[0] = u32x4{};
      if (kt + wkey + 8 + lkey >= n_k) kr[1] = vr[1] = u32x4{};
    }
  };
  // V is staged as fp16: the weights of the P.V product are fp16.
  auto convert_v = [&](const u32x4 (&vr)[2], u32x4 (&v16)[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) v16[u][e] = bf16x2_to_f16x2(vr[u][e]);
  };
  auto write_tile = [&](int stage, const u32x4 (&kr)[2], const u32x4 (&v16)[2]) {
    uint8_t* ks = smem + stage * 2 * kTileBytes;
    uint8_t* vs = ks + kTileBytes;
    *reinterpret_cast<u32x4*>(ks + tile_swizzle(wkey + lkey, ld_c)) = kr[0];
    *reinterpret_cast<u32x4*>(ks + tile_swizzle(wkey + 8 + lkey, ld_c)) = kr[1];
    *reinterpret_cast<u32x4*>(vs + tile_swizzle(wkey + lkey, ld_c)) = v16[0];
    *reinterpret_cast<u32x4*>(vs + tile_swizzle(wkey + 8 + lkey, ld_c)) = v16[1];
  };

  int pid = 0;
  {
    u32x4 kr[2], vr[2], v16[2];
    if (PAGED) pid = page_of(k_first);
    load_tile(k_first, pid, kr, vr);
    if (PAGED) pid = page_of(k_first + kBN);
    fix_tail(k_first, kr, vr);
    convert_v(vr, v16);
    write_tile(0, kr, v16);
  }
  __syncthreads();

  // Lane addresses of the operand reads in stage 0; the stage and the half
  // tile are compile-time offsets added by the read instructions themselves.
  uint32_t k_lane[4], v_lane[2][2];
#pragma unroll
  for (int kstep = 0; kstep < 4; ++kstep) k_lane[kstep] = opaque(smem0 + tl.k[kstep]);
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    v_lane[db][0] = opaque(smem0 + kTileBytes + tl.v[db][0]);
    v_lane[db][1] = opaque(smem0 + kTileBytes + tl.v[db][1]);
  }

  // One key tile; STAGE (the LDS buffer holding it) is a compile-time
  // constant, so the tile loop below is unrolled by two.
  auto tile_step = [&](const int it, auto stage_c) {
    constexpr int STAGE = decltype(stage_c)::value;
    constexpr uint32_t st = STAGE * 2 * kTileBytes;
    const int kt = k_first + it * kBN;
    u32x4 kr[2], vr[2], v16[2];
    const bool more = it + 1 < ntiles;
    bool converted = false;   // the next tile's V already converted (uniform)
    if (more) {
      load_tile(kt + kBN, pid, kr, vr);
      if (PAGED) pid = page_of(kt + 2 * kBN);
    }

    const bool wave_skip = !wave_live || kt > wp_max || (W > 0 && kt + kBN - 1 < wp_min - W + 1);
    if (!wave_skip) {
      const bool need_mask = (kt + kBN - 1 > wp_min) || (W > 0 && kt < wp_max - W + 1);
      // The tile is processed as two 32-key halves, pipelined inside the
      // wave so that matrix and vector instructions stay independent and can
      // issue side by side:
      //   S0 | S1 with weights(S0) | P0.V0 with weights(S1) | P1.V1
      // Element i of s[rb] (half kb) is key kt + 32*kb + 8*(i/4) + 4*half + i%4
      // against row r32 + 32*rb.
      auto read_k = [&](int kb, bf16x8 (&kop)[4]) {
#pragma unroll
        for (int kstep = 0; kstep < 4; ++kstep)
          kop[kstep] = *lds_at<const bf16x8>(k_lane[kstep] + (st + kb * 32 * 128));
      };
      auto mma_scores = [&](const bf16x8 (&kop)[4], f32x16 (&sh)[2]) {
        sh[0] = f32x16{};
        sh[1] = f32x16{};
#pragma unroll
        for (int kstep = 0; kstep < 4; ++kstep) {
          sh[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kstep], qop[0][kstep], sh[0], 0, 0, 0);
          sh[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kstep], qop[1][kstep], sh[1], 0, 0, 0);
        }
      };
      auto mask_half = [&](int kb, f32x16 (&sh)[2]) {
        // a real (scalar) branch: only tiles on the diagonal or the window edge pay for it
        __asm__ volatile("");
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int hi_off = my_p[rb] - kt - 32 * kb - 4 * half;
          const int lo_off = W > 0 ? my_lo[rb] - kt - 32 * kb - 4 * half : -kBN;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int off = 8 * (i >> 2) + (i & 3);
            sh[rb][i] = (off <= hi_off && off >= lo_off) ? sh[rb][i] : kNegInf;
          }
        }
      };
      auto read_v = [&](int kb, f16x8 (&vt)[2][2]) {   // [hh][db]
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const uint32_t vlo = v_lane[db][0] + st;
          const uint32_t vhi = v_lane[db][1] + st;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int r = 2 * kb + hh;
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_at<i16x4>(vlo + r * 16 * 128));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_at<i16x4>(vhi + r * 16 * 128));
            typedef __attribute__((ext_vector_type(8))) short i16x8;
            vt[hh][db] = __builtin_bit_cast(f16x8, i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
          }
        }
      };
      auto mma_pv = [&](const f16x8 (&vt)[2][2], const f16x8 (&pop)[2][2]) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int db = 0; db < 2; ++db) {
            acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vt[hh][db], pop[0][hh], acc[0][db], 0, 0, 0);
            acc[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vt[hh][db], pop[1][hh], acc[1][db], 0, 0, 0);
          }
      };
      // rare path of a half (a key far above the reference): recompute its
      // scores from the staged tile, move the reference to the row maxima,
      // rescale, and redo the weights
      auto rebase = [&](int kb, f16x8 (&pop)[2][2], float (&tsum)[2]) {
        __asm__ volatile("");
        bf16x8 kop[4];
        read_k(kb, kop);
        f32x16 sh[2];
        mma_scores(kop, sh);
        reads_then_mfmas<4, 8>();
        if (need_mask) mask_half(kb, sh);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          float mx = sh[rb][0];
#pragma unroll
          for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sh[rb][i]);
          mx = fmaxf(mx, shfl_xor_f32(mx, 32));
          const float m_new = fmaxf(m[rb], mx * c);
          const float alpha = exp2_hw(m[rb] - m_new);
          m[rb] = m_new;
          dsum[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[rb][db][i] *= alpha;
        }
        half_weights(sh, m, c, pop, tsum);
      };

      f32x16 s0[2], s1[2];
      f16x8 p0[2][2], p1[2][2];
      float t0s[2], t1s[2];
      // Every step's LDS operands are read one step ahead: both K halves
      // before S0, V0 at the start of S1's step, V1 at the start of P0.V0's,
      // so no step waits on its own reads.
      bf16x8 k0[4], k1[4];
      read_k(0, k0);
      read_k(1, k1);
      mma_scores(k0, s0);
      reads_then_mfmas<8, 8>();
      if (need_mask) mask_half(0, s0);
      if (it == 0) {
        // the workgroup's first key tile: the reference goes to the row
        // maxima of its first half before any weight is taken (from
        // -FLT_MAX every weight would overflow and the half be redone);
        // acc and the denominator are still zero, so nothing is rescaled
        __asm__ volatile("");
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          float mx = s0[rb][0];
#pragma unroll
          for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s0[rb][i]);
          mx = fmaxf(mx, shfl_xor_f32(mx, 32));
          m[rb] = fmaxf(m[rb], mx * c);
        }
      }
      // The two overlapped steps are interleaved by hand: each MFMA is
      // followed by four weights of the other half (fma, exp2, pack), and
      // scheduling fences keep the compiler from regrouping them, so the
      // wave issues vector work while its matrix product runs.
      f16x8 v0[2][2];
      read_v(0, v0);
      {
        f16x2 h[2][8];
        s1[0] = f32x16{};
        s1[1] = f32x16{};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int kstep = u >> 1, rb = u & 1;
          s1[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1[kstep], qop[rb][kstep], s1[rb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          weight_pair(s0, m, c, u >> 2, 2 * (u & 3), h);
          weight_pair(s0, m, c, u >> 2, 2 * (u & 3) + 1, h);
          __builtin_amdgcn_sched_barrier(0);
        }
        finish_weights(h, p0, t0s);
      }
      if ((__builtin_amdgcn_ballot_w64(t0s[0] > kSumLimit) | __builtin_amdgcn_ballot_w64(t0s[1] > kSumLimit)) != 0)
        rebase(0, p0, t0s);
      dsum[0] += t0s[0];
      dsum[1] += t0s[1];
      if (need_mask) mask_half(1, s1);
      f16x8 v1[2][2];
      read_v(1, v1);
      {
        f16x2 h[2][8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int hh = u >> 2, db = (u >> 1) & 1, rb = u & 1;
          acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v0[hh][db], p0[rb][hh], acc[rb][db], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          weight_pair(s1, m, c, u >> 2, 2 * (u & 3), h);
          weight_pair(s1, m, c, u >> 2, 2 * (u & 3) + 1, h);
          __builtin_amdgcn_sched_barrier(0);
        }
        finish_weights(h, p1, t1s);
      }
      if ((__builtin_amdgcn_ballot_w64(t1s[0] > kSumLimit) | __builtin_amdgcn_ballot_w64(t1s[1] > kSumLimit)) != 0)
        rebase(1, p1, t1s);
      dsum[0] += t1s[0];
      dsum[1] += t1s[1];
      if (more) {
        // the last product of the tile carries the conversion of the next
        // tile's V: one dword of it after each MFMA
        fix_tail(kt + kBN, kr, vr);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int hh = u >> 2, db = (u >> 1) & 1, rb = u & 1;
          acc[rb][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v1[hh][db], p1[rb][hh], acc[rb][db], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          v16[u >> 2][u & 3] = bf16x2_to_f16x2(vr[u >> 2][u & 3]);
          __builtin_amdgcn_sched_barrier(0);
        }
        converted = true;
      } else {
        mma_pv(v1, p1);
      }
    }

    if (more) {
      if (!converted) {
        fix_tail(kt + kBN, kr, vr);
        convert_v(vr, v16);
      }
      write_tile(STAGE ^ 1, kr, v16);
    }
    __syncthreads();
  };
  for (int it = 0; it < ntiles; it += 2) {
    tile_step(it, std::integral_constant<int, 0>{});
    if (it + 1 < ntiles) tile_step(it + 1, std::integral_constant<int, 1>{});
  }

  if (!wave_live) return;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float d = dsum[rb] + shfl_xor_f32(dsum[rb], 32);
    if (my_t[rb] >= n_q) continue;
    float lse2;
    // every real row sees its own key, so d > 0 here
    const float inv = fold_sink(sink2, d > 0.f ? m[rb] : kNegInf, d, &lse2);
    const size_t orow = ((size_t)(q_begin + my_t[rb]) * a.num_qo_heads + head) * kHeadDim;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * db + 8 * q4 + 4 * half;
        u32x2 w;
        w[0] = pack_bf16x2(acc[rb][db][4 * q4 + 0] * inv, acc[rb][db][4 * q4 + 1] * inv);
        w[1] = pack_bf16x2(acc[rb][db][4 * q4 + 2] * inv, acc[rb][db][4 * q4 + 3] * inv);
        *reinterpret_cast<u32x2*>(a.out + orow + d0) = w;
      }
    if (a.lse != nullptr && half == 0)
      a.lse[(size_t)(q_begin + my_t[rb]) * a.num_qo_heads + head] = lse2 * kLn2;
  }
}

}  // namespace

// Heads per workgroup: four when the GQA group splits into fours, else one.
static int heads_per_workgroup(int32_t group) { return group % 4 == 0 ? 4 : 1; }

template <bool PLANNED>
static void launch_shape(const PrefillArgs& a, const PlanArg<PLANNED>& plan, int hp, dim3 grid,
                         hipStream_t stream) {
  const dim3 block(kWaves * 64);
  if (a.paged) {
    if (hp == 4) hipLaunchKernelGGL((prefill_kernel<true, 4, PLANNED>), grid, block, 0, stream, a, plan);
    else hipLaunchKernelGGL((prefill_kernel<true, 1, PLANNED>), grid, block, 0, stream, a, plan);
  } else {
    if (hp == 4) hipLaunchKernelGGL((prefill_kernel<false, 4, PLANNED>), grid, block, 0, stream, a, plan);
    else hipLaunchKernelGGL((prefill_kernel<false, 1, PLANNED>), grid, block, 0, stream, a, plan);
  }
}

hipError_t launch_prefill(const PrefillArgs& a, const PrefillPlan* plan, hipStream_t stream) {
  const int hp = heads_per_workgroup(a.group);
  const long blocks = (long)a.num_slots * (a.num_qo_heads / hp);
  if (blocks <= 0) return hipSuccess;
  if (plan != nullptr && a.num_slots > kPrefillPlanMax) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks);
  if (plan != nullptr) launch_shape<true>(a, PlanArg<true>{*plan}, hp, grid, stream);
  else launch_shape<false>(a, PlanArg<false>{0}, hp, grid, stream);
  return hipGetLastError();
}

int prefill_rows_per_tile(int32_t window, int32_t group) {
  (void)window;
  return kRowsPerWave * (kWaves / heads_per_workgroup(group));
}

}  // namespace sinkattn
