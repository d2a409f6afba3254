// Append new keys/values to a paged KV cache with rotary position embedding
// applied to the new queries and keys.
//
// Sources: "GPT-OSS on day 0", section "GPT-OSS on Hopper" (the models use
// YaRN rotary position encoding); "Accelerating Sonar through speculation",
// section "Inference with speculative decoding" (per-request KV pages, page
// tables built on the CPU).  The pages give neither the YaRN constants nor the
// pair layout: the angles come from a caller-supplied cos/sin table (so any
// frequency scaling lives there) and the pair layout is a flag.
//
// One wave per appended token: it finds its request (binary search over the
// append offsets), the token's position kv_len - n + i and its page slot, then
// streams the token's query heads, key heads and value heads, eight 64-dim
// rows per pass (eight lanes a row).  Each lane holds whole rotation pairs:
// dims {4m..4m+3} and {32+4m..32+4m+3} in the half layout, {8m..8m+7} in the
// interleaved one, so no lane exchange is needed.  Pure data movement:
// memory-bound.

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace sinkattn {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)to_bf16_bits(lo) | ((uint32_t)to_bf16_bits(hi) << 16);
}

__global__ __launch_bounds__(256) void append_rope_kernel(AppendArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.total_new) return;                 // uniform per wave

  // request of token t: the last b with append_indptr[b] <= t
  int lo = 0, hi = a.batch;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.append_indptr[mid] <= t) lo = mid;
    else hi = mid;
  }
  const int b = lo;
  const int first = a.append_indptr[b];
  const int n_b = a.append_indptr[b + 1] - first;
  const int pos = a.kv_len[b] - n_b + (t - first);
  if (pos < 0 || pos >= a.max_pos) return;      // outside the table: nothing is written
  const int page = a.page_indices[a.page_indptr[b] + pos / kPageSize];
  const int slot = pos % kPageSize;

  const int m = lane & 7;                       // this lane's pairs: 4m .. 4m+3
  const f32x4 c = *reinterpret_cast<const f32x4*>(a.cos_sin + (size_t)pos * kHeadDim + 4 * m);
  const f32x4 s = *reinterpret_cast<const f32x4*>(a.cos_sin + (size_t)pos * kHeadDim + 32 + 4 * m);

  const int nq = a.q != nullptr ? a.num_qo_heads : 0;
  const int units = nq + 2 * a.num_kv_heads;
  for (int u = lane >> 3; u < units; u += 8) {
    const uint16_t* src;
    uint16_t* dst;
    bool rot = true;
    if (u < nq) {
      src = a.q + ((size_t)t * a.num_qo_heads + u) * kHeadDim;
      dst = a.q_out + ((size_t)t * a.num_qo_heads + u) * kHeadDim;
    } else if (u < nq + a.num_kv_heads) {
      const int h = u - nq;
      src = a.k_new + ((size_t)t * a.num_kv_heads + h) * kHeadDim;
      dst = a.k_pool + (((size_t)page * a.num_kv_heads + h) * kPageSize + slot) * kHeadDim;
    } else {
      const int h = u - nq - a.num_kv_heads;
      src = a.v_new + ((size_t)t * a.num_kv_heads + h) * kHeadDim;
      dst = a.v_pool + (((size_t)page * a.num_kv_heads + h) * kPageSize + slot) * kHeadDim;
      rot = false;
    }
    if (a.interleaved) {
      u32x4 x = *reinterpret_cast<const u32x4*>(src + 8 * m);   // pairs (2f, 2f+1), f = 4m + e
      if (rot) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x1 = bf16_lo(x[e]), x2 = bf16_hi(x[e]);
          x[e] = pack_bf16(x1 * c[e] - x2 * s[e], x2 * c[e] + x1 * s[e]);
        }
      }
      *reinterpret_cast<u32x4*>(dst + 8 * m) = x;
    } else {
      u32x2 x = *reinterpret_cast<const u32x2*>(src + 4 * m);        // dims 4m .. 4m+3
      u32x2 y = *reinterpret_cast<const u32x2*>(src + 32 + 4 * m);   // their partners
      if (rot) {
        const float x0 = bf16_lo(x[0]), x1 = bf16_hi(x[0]), x2 = bf16_lo(x[1]), x3 = bf16_hi(x[1]);
        const float y0 = bf16_lo(y[0]), y1 = bf16_hi(y[0]), y2 = bf16_lo(y[1]), y3 = bf16_hi(y[1]);
        x[0] = pack_bf16(x0 * c[0] - y0 * s[0], x1 * c[1] - y1 * s[1]);
        x[1] = pack_bf16(x2 * c[2] - y2 * s[2], x3 * c[3] - y3 * s[3]);
        y[0] = pack_bf16(y0 * c[0] + x0 * s[0], y1 * c[1] + x1 * s[1]);
        y[1] = pack_bf16(y2 * c[2] + x2 * s[2], y3 * c[3] + x3 * s[3]);
      }
      *reinterpret_cast<u32x2*>(dst + 4 * m) = x;
      *reinterpret_cast<u32x2*>(dst + 32 + 4 * m) = y;
    }
  }
}

}  // namespace

hipError_t launch_append_rope(const AppendArgs& a, hipStream_t stream) {
  if (a.total_new <= 0) return hipSuccess;
  hipLaunchKernelGGL(append_rope_kernel, dim3((unsigned)((a.total_new + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sinkattn
