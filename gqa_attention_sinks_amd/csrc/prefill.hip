// Causal / sliding-window prefill with per-head attention sinks.
//
// Method: Perplexity blog "GPT-OSS on day 0" (French rendering "GPT-OSS au
// jour J"), section "Kernels for GPT-OSS > Sink attention": the sink is one
// more term of the softmax; the streaming softmax (running max m, scale d)
// starts from (sink, 1), so the sink costs nothing per key.
//
// Work decomposition (gfx950):
//   workgroup = (tile of 256 query rows of one request, one query head);
//   4 waves x 64 query rows (two 32-row MFMA blocks, so every K/V operand
//   read from LDS feeds two MFMAs).  Consecutive workgroup ids walk the KV heads
//   first, so with 8 KV heads and 8 XCDs each XCD's L2 serves one KV head.
//   Tiles of a request are issued longest first (causal work grows with the
//   row index).
//   Per KV tile of 64 keys (K and V staged in LDS, double buffered, 16-byte
//   chunks XOR-swizzled by key):
//     S^T[64 keys x 64 rows] = K . Q^T    -> 16 x MFMA 32x32x16 bf16 (Q^T in registers)
//     base-2 online softmax on the accumulator: each lane holds two query
//     rows and 32 of their keys, so a row max needs one exchange with
//     lane ^ 32; the reference max moves lazily (only when a row max exceeds
//     it by 2^8), so most tiles skip rescaling the accumulators
//     O^T[64 dims x 64 rows] += V^T . P^T -> 16 x MFMA 32x32x16 fp16
//       (P^T is the score accumulator converted to fp16; V is converted to
//        fp16 once when its tile is staged, and V^T comes from the natural
//        [key][dim] LDS tile through ds_read_b64_tr_b16).  fp16 weights carry
//        three more mantissa bits than bf16; they are taken relative to the
//        running key maximum and the sink is folded in at the end, which
//        gives exactly the state of the sink-seeded recurrence.
//   Masking is applied only on tiles that cross the causal diagonal or the
//   window's lower edge.

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace sinkattn {
namespace {

constexpr int kWaves = 4;
constexpr int kRowsPerWave = 64;               // two 32-row MFMA blocks per wave
constexpr int kBM = kWaves * kRowsPerWave;     // query rows per workgroup
constexpr int kBN = 64;                        // keys per tile
constexpr float kLazy = 8.f;                   // log2 slack before the running max moves
constexpr int kTileBytes = kBN * kHeadDim * 2;   // 8 KiB

typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;

__device__ __forceinline__ int tile_swizzle(int key, int chunk) {
  return key * 128 + ((chunk ^ (key & 7)) << 4);
}

__device__ __forceinline__ u32x4 ldg16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Wave priority around MFMA clusters: while one wave of a SIMD issues its
// matrix instructions, the other wave's vector instructions fill the gaps.
__device__ __forceinline__ void mfma_phase_begin() {
#if SINKATTN_PREFILL_SETPRIO
  __builtin_amdgcn_s_setprio(1);
#endif
}
__device__ __forceinline__ void mfma_phase_end() {
#if SINKATTN_PREFILL_SETPRIO
  __builtin_amdgcn_s_setprio(0);
#endif
}

template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds_ptr(uint8_t* p) {
  return (__attribute__((address_space(3))) T*)(p);
}

// Find the (request, tile) handled by tile slot `slot`: tiles are numbered
// request by request; every thread sums a run of requests, then a block scan.
__device__ bool locate_tile(const PrefillArgs& a, int slot, int* s_scan, int* out_b, int* out_tile) {
  const int tid = threadIdx.x;
  const int per = (a.batch + kWaves * 64 - 1) / (kWaves * 64);
  const int b0 = min(tid * per, a.batch);
  const int b1 = min(b0 + per, a.batch);
  int local = 0;
  for (int b = b0; b < b1; ++b) {
    const int n = a.qo_indptr[b + 1] - a.qo_indptr[b];
    if (!(a.skip_single_rows && n == 1)) local += (n + kBM - 1) / kBM;
  }
  s_scan[tid] = local;
  __syncthreads();
  for (int off = 1; off < kWaves * 64; off <<= 1) {
    const int v = tid >= off ? s_scan[tid - off] : 0;
    __syncthreads();
    s_scan[tid] += v;
    __syncthreads();
  }
  const int excl = s_scan[tid] - local;
  __shared__ int s_found[2];
  if (tid == 0) s_found[0] = -1;
  __syncthreads();
  if (slot >= excl && slot < excl + local) {
    int base = excl;
    for (int b = b0; b < b1; ++b) {
      const int n = a.qo_indptr[b + 1] - a.qo_indptr[b];
      const int nt = (a.skip_single_rows && n == 1) ? 0 : (n + kBM - 1) / kBM;
      if (slot < base + nt) {
        s_found[0] = b;
        s_found[1] = nt - 1 - (slot - base);   // longest tile first
        break;
      }
      base += nt;
    }
  }
  __syncthreads();
  *out_b = s_found[0];
  *out_tile = s_found[1];
  return s_found[0] >= 0;
}

template <bool PAGED>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillArgs a) {
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
  const int hg = id % a.group;
  const int slot = id / a.group;
  const int head = g * a.group + hg;

  int b, tile;
  if (!locate_tile(a, slot, s_scan, &b, &tile)) return;
  b = __builtin_amdgcn_readfirstlane(b);
  tile = __builtin_amdgcn_readfirstlane(tile);

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
  const int t0 = tile * kBM;
  const int t_last = min(t0 + kBM, n_q) - 1;
  const int W = a.window;
  const int lo_first = W > 0 ? max(0, shift + t0 - W + 1) : 0;
  const int k_first = (lo_first / kBN) * kBN;
  const int k_end = shift + t_last + 1;   // exclusive
  const int ntiles = (k_end - k_first + kBN - 1) / kBN;

  // this wave's 64 rows (two 32-row MFMA blocks) and the two rows of this lane
  const int wt0 = t0 + kRowsPerWave * wave;
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

  // Key-domain streaming state per row: running max reference m (base 2; may
  // lag the true key maximum by up to kLazy), this lane's part of the
  // denominator, and the P.V accumulator.  The sink is folded in at the end
  // (fold_sink), which yields the state of the sink-seeded recurrence.
  float m[2] = {kNegInf, kNegInf}, dsum[2] = {0.f, 0.f};
  f32x16 acc[2][2] = {};   // [row block][dim block]
  const float c = a.scale_log2;

  // tile loader: thread -> (key = tid / 4, 32 bytes at dims 16 * (tid % 4))
  const int ld_key = tid >> 2;
  const int ld_c = (tid & 3) * 2;   // first 16-byte chunk
  const size_t g_off = (size_t)g * (PAGED ? kPageSize * kHeadDim : kHeadDim) + ld_c * 8;
  const int32_t* page_list = PAGED ? a.page_indices + a.kv_indptr[b] : nullptr;
  // paged: id of the page holding this thread's key, fetched one tile ahead
  auto page_of = [&](int kt) -> int {
    return page_list[min(kt + ld_key, n_k - 1) / kPageSize];
  };
  int pid = 0;
  auto load_rows = [&](int key, int page, u32x4 (&kr)[2], u32x4 (&vr)[2]) {
    size_t row;
    if (PAGED) row = ((size_t)page * a.num_kv_heads * kPageSize + key % kPageSize) * kHeadDim + g_off;
    else row = (size_t)(kv_begin + key) * a.num_kv_heads * kHeadDim + g_off;
    const uint16_t* kp = a.k + row;
    const uint16_t* vp = a.v + row;
    kr[0] = ldg16(kp);
    kr[1] = ldg16(kp + 8);
    vr[0] = ldg16(vp);
    vr[1] = ldg16(vp + 8);
  };
  // rows past the last key read the last key's row (always in bounds) and are
  // zeroed when staged, so the common full tile carries no per-row checks
  auto load_tile = [&](int kt, int page, u32x4 (&kr)[2], u32x4 (&vr)[2]) {
    load_rows(min(kt + ld_key, n_k - 1), page, kr, vr);
  };
  auto store_tile = [&](int stage, int kt, u32x4 (&kr)[2], u32x4 (&vr)[2]) {
    uint8_t* ks = smem + stage * 2 * kTileBytes;
    uint8_t* vs = ks + kTileBytes;
    if (kt + kBN > n_k) {           // uniform: only the last tile of the range
      __asm__ volatile("");
      if (kt + ld_key >= n_k) kr[0] = kr[1] = vr[0] = vr[1] = u32x4{};
    }
    *reinterpret_cast<u32x4*>(ks + tile_swizzle(ld_key, ld_c)) = kr[0];
    *reinterpret_cast<u32x4*>(ks + tile_swizzle(ld_key, ld_c + 1)) = kr[1];
    // V is staged as fp16: the weights of the P.V product are fp16
    u32x4 v16[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) v16[u][e] = bf16x2_to_f16x2(vr[u][e]);
    *reinterpret_cast<u32x4*>(vs + tile_swizzle(ld_key, ld_c)) = v16[0];
    *reinterpret_cast<u32x4*>(vs + tile_swizzle(ld_key, ld_c + 1)) = v16[1];
  };

  {
    u32x4 kr[2], vr[2];
    if (PAGED) pid = page_of(k_first);
    load_tile(k_first, pid, kr, vr);
    if (PAGED) pid = page_of(k_first + kBN);
    store_tile(0, k_first, kr, vr);
  }
  __syncthreads();

  const int j16 = lane & 15;
  const int gr_odd = (lane >> 4) & 1;

  for (int it = 0; it < ntiles; ++it) {
    const int kt = k_first + it * kBN;
    u32x4 kr[2], vr[2];
    const bool more = it + 1 < ntiles;
    if (more) {
      load_tile(kt + kBN, pid, kr, vr);
      if (PAGED) pid = page_of(kt + 2 * kBN);
    }

    const bool wave_skip = !wave_live || kt > wp_max || (W > 0 && kt + kBN - 1 < wp_min - W + 1);
    if (!wave_skip) {
      uint8_t* ks = smem + (it & 1) * 2 * kTileBytes;
      uint8_t* vs = ks + kTileBytes;
      // S^T = K . Q^T : [key block][row block]
      f32x16 s[2][2];
      // all eight K operands are read before the first MFMA, so the LDS
      // latency is paid once per tile rather than once per MFMA pair
      bf16x8 kop[2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int kstep = 0; kstep < 4; ++kstep)
          kop[kb][kstep] = *reinterpret_cast<const bf16x8*>(ks + tile_swizzle(32 * kb + r32, 2 * kstep + half));
      mfma_phase_begin();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb][0] = f32x16{};
        s[kb][1] = f32x16{};
#pragma unroll
        for (int kstep = 0; kstep < 4; ++kstep) {
          s[kb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kb][kstep], qop[0][kstep], s[kb][0], 0, 0, 0);
          s[kb][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kb][kstep], qop[1][kstep], s[kb][1], 0, 0, 0);
        }
      }
      mfma_phase_end();
#if SINKATTN_PREFILL_SCHED
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // the eight K reads
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);  // then the sixteen MFMAs
#endif
      // causal diagonal / window edge: element i of key block kb is key
      // kt + 32*kb + 8*(i/4) + 4*half + i%4
      const bool need_mask = (kt + kBN - 1 > wp_min) || (W > 0 && kt < wp_max - W + 1);
      if (need_mask) {
        // a real (scalar) branch: only tiles on the diagonal or the window edge pay for it
        __asm__ volatile("");
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const int hi_off = my_p[rb] - kt - 4 * half;
          const int lo_off = W > 0 ? my_lo[rb] - kt - 4 * half : -kBN;
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int off = 32 * kb + 8 * (i >> 2) + (i & 3);
              s[kb][rb][i] = (off <= hi_off && off >= lo_off) ? s[kb][rb][i] : kNegInf;
            }
        }
      }
      // row maxima; the reference max moves only when a row's max exceeds it
      // by more than kLazy (weights stay <= 2^kLazy), so most tiles skip the
      // rescale of the accumulators
      float cand[2];
      bool grow = false;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        // a running chain compiles to one v_max3 per two values
        float mx = s[0][rb][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[0][rb][i]);
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[1][rb][i]);
        mx = fmaxf(mx, shfl_xor_f32(mx, 32));
        cand[rb] = mx * c;
        grow |= cand[rb] > m[rb] + kLazy;
      }
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        __asm__ volatile("");
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          const float m_new = cand[rb] > m[rb] + kLazy ? cand[rb] : m[rb];
          const float alpha = (m_new == m[rb]) ? 1.f : exp2_hw(m[rb] - m_new);
          m[rb] = m_new;
          dsum[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < 2; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[rb][db][i] *= alpha;
        }
      }
      // V^T operands for the P.V product, read from LDS before the weights
      // are computed so their latency hides behind the vector work
      f16x8 vtop[4][2];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key_a = 16 * r + 4 * half + (j16 >> 2);
        const int key_b = key_a + 8;
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const int chunk = 4 * db + 2 * gr_odd + ((j16 & 3) >> 1);
          const int sub = 8 * (j16 & 1);
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<i16x4>(vs + tile_swizzle(key_a, chunk) + sub));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(lds_ptr<i16x4>(vs + tile_swizzle(key_b, chunk) + sub));
          typedef __attribute__((ext_vector_type(8))) short i16x8;
          vtop[r][db] = __builtin_bit_cast(f16x8, i16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
        }
      }
      // P^T operands (fp16): operand r covers keys 16r .. 16r+15 of the tile
      f16x8 pop[2][4];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float m_use = m[rb] == kNegInf ? 0.f : m[rb];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pv[e] = exp2_hw(__builtin_fmaf(s[kb][rb][8 * hh + e], c, -m_use));
            u32x4 pk;
            pk[0] = pack_f16x2(pv[0], pv[1]);
            pk[1] = pack_f16x2(pv[2], pv[3]);
            pk[2] = pack_f16x2(pv[4], pv[5]);
            pk[3] = pack_f16x2(pv[6], pv[7]);
#pragma unroll
            for (int e = 0; e < 4; ++e) dsum[rb] = add_f16x2(pk[e], dsum[rb]);
            pop[rb][2 * kb + hh] = __builtin_bit_cast(f16x8, pk);
          }
      }
      // O^T += V^T . P^T ; each V^T operand feeds both row blocks
      mfma_phase_begin();
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vtop[r][db], pop[0][r], acc[0][db], 0, 0, 0);
          acc[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vtop[r][db], pop[1][r], acc[1][db], 0, 0, 0);
        }
      mfma_phase_end();
    }

    if (more) store_tile((it + 1) & 1, kt + kBN, kr, vr);
    __syncthreads();
  }

  if (!wave_live) return;
  const float sink2 = a.sinks != nullptr ? a.sinks[head] * kLog2e : kNegInf;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const float d = dsum[rb] + shfl_xor_f32(dsum[rb], 32);
    if (my_t[rb] >= n_q) continue;
    float lse2;
    const float inv = fold_sink(sink2, m[rb], d, &lse2);
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

hipError_t launch_prefill(const PrefillArgs& a, int32_t total_q, hipStream_t stream) {
  (void)total_q;
  const long blocks = (long)a.num_slots * a.num_qo_heads;
  if (blocks <= 0) return hipSuccess;
  if (a.paged)
    hipLaunchKernelGGL(prefill_kernel<true>, dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream, a);
  else
    hipLaunchKernelGGL(prefill_kernel<false>, dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream, a);
  return hipGetLastError();
}

int prefill_rows_per_tile() { return kBM; }

}  // namespace sinkattn
