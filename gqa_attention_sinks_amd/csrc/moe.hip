// MoE routing weights: the top-K experts of each token and the softmax over
// their logits alone.
//
// Source: "GPT-OSS on day 0", sections "GPT-OSS on Hopper" (softmax after the
// top-K selection for the expert weights) and "Kernels for GPT-OSS > MoE"
// (GPT-OSS takes the softmax over the top-K selected experts only, not over
// all experts as DeepSeek-style models do, and the expert weights must be
// computed in bfloat16 precision).
//
// One wave per token.  Each logit becomes a 32-bit key: the bf16 bits mapped
// to an unsigned order (larger logit, larger key) in the high half and the
// complemented expert index in the low half, so one unsigned max picks the
// largest logit and, among equal logits, the lowest index.  K rounds of a
// wave-wide max (six xor exchanges) select the experts in order; the selected
// key is then cleared.  The softmax over the K selected bf16 logits runs in
// fp32 and is rounded to bf16.

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace sinkattn {
namespace {

constexpr int kMoeMaxPerLane = 8;   // experts per lane: up to 512 experts

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int mask) {
  const int src = __lane_id() ^ mask;
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)v);
}

__device__ __forceinline__ uint32_t order_key(uint16_t bits, int expert) {
  if (bits == 0x8000u) bits = 0;   // -0 equals +0: the same key, so the index decides
  // sign-magnitude -> unsigned order: negatives reversed below positives
  const uint32_t ord = (bits & 0x8000u) ? (uint32_t)(~bits & 0xffffu) : (uint32_t)(bits | 0x8000u);
  return (ord << 16) | (uint32_t)(0xffff - expert);
}

__global__ __launch_bounds__(256) void moe_topk_softmax_kernel(MoeArgs a) {
  const int lane = threadIdx.x & 63;
  const long t = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= a.num_tokens) return;                 // uniform per wave
  const uint16_t* row = a.logits + t * a.num_experts;
  uint32_t key[kMoeMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMoeMaxPerLane; ++i) {
    const int e = i * 64 + lane;
    key[i] = e < a.num_experts ? order_key(row[e], e) : 0u;   // 0: below every real key
  }
  float sel_logit = 0.f;   // lane r < K keeps the r-th selected logit
  int sel_idx = 0;
  for (int r = 0; r < a.top_k; ++r) {
    uint32_t best = 0u;
#pragma unroll
    for (int i = 0; i < kMoeMaxPerLane; ++i) best = max(best, key[i]);
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) best = max(best, shfl_xor_u32(best, m));
    const int e = 0xffff - (int)(best & 0xffffu);
    // clear the winner (its key is unique: the index is in it)
#pragma unroll
    for (int i = 0; i < kMoeMaxPerLane; ++i)
      if (key[i] == best) key[i] = 0u;
    if (lane == r) {
      sel_idx = e;
      sel_logit = __builtin_bit_cast(float, (uint32_t)row[e] << 16);
    }
  }
  // softmax over the selected logits (lanes 0 .. K-1); the first is the largest
  const float top = __builtin_bit_cast(float, (uint32_t)__builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, sel_logit)));
  float ex = lane < a.top_k ? exp2_hw((sel_logit - top) * kLog2e) : 0.f;
  float sum = ex;
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) sum += shfl_xor_f32(sum, m);   // K <= 8: lanes 0..7 hold every term
  if (lane < a.top_k) {
    a.topk_idx[t * a.top_k + lane] = sel_idx;
    a.topk_w[t * a.top_k + lane] = to_bf16_bits(ex / sum);
  }
}

}  // namespace

hipError_t launch_moe_topk_softmax(const MoeArgs& a, hipStream_t stream) {
  if (a.num_tokens <= 0) return hipSuccess;
  hipLaunchKernelGGL(moe_topk_softmax_kernel, dim3((unsigned)((a.num_tokens + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sinkattn
