// MoE routing weights: the top-K experts of each token and the softmax over
// their logits alone.
//
// Source: "GPT-OSS on day 0", sections "GPT-OSS on Hopper" (softmax after the
// top-K selection for the expert weights) and "Kernels for GPT-OSS > MoE"
// (GPT-OSS takes the softmax over the top-K selected experts only, not over
// all experts as DeepSeek-style models do, and the expert weights must be
// computed in bfloat16 precision).
//
// L lanes per token (four up to 256 experts, else eight).  Each logit becomes a
// 32-bit key: the bf16 bits mapped to an unsigned order (larger logit, larger
// key; -0 and +0 the same) in the high half and the complemented expert index
// in the low half, so one unsigned comparison orders by logit and, among equal
// logits, puts the lower index first.  Each lane keeps the top KP keys of its
// own experts in a descending register list; inserting a key costs one
// three-input median per list entry (entry i becomes the median of the old
// entries i - 1 and i and the key), and the map needs no compare-and-select,
// so the loop is plain integer arithmetic.  log2(L) exchange levels (lanes
// 1, 2, 4 apart) merge the L lists: the elementwise max of a list and its
// partner's reversed list holds the top KP of both, and a bitonic network
// sorts it.  Every lane then holds the token's top KP; lane s writes picks
// s, s + L, ... (ids and weights), the softmax over the K selected bf16
// logits evaluated in fp32 and rounded to bf16.

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace sinkattn {
namespace {

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int mask) {
  const int src = __lane_id() ^ mask;
  return (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)v);
}

// Order key of a logit whose bf16 bits sit in the high half of x (low half
// zero), with idx = 0xffff - expert added in the low half.  A non-negative
// value v maps to v + 2^31, a negative one to -v (two's complement, below
// 2^31), so the map is monotone and -0 lands on +0's key.
__device__ __forceinline__ uint32_t order_key(uint32_t x, uint32_t idx) {
  const uint32_t s = (uint32_t)((int32_t)x >> 31);   // all ones for a negative value
  return (((x ^ s) - s) ^ (~s & 0x80000000u)) + idx;
}

// The same map on both bf16 halves of w at once (16-bit lanes): the high
// halves of the two keys, in the low and high half of the result.
typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2 order_hi_pair(uint32_t w) {
  const u16x2 b = __builtin_bit_cast(u16x2, w);
  const u16x2 s = __builtin_bit_cast(u16x2, __builtin_bit_cast(s16x2, b) >> (short)15);
  return ((b ^ s) - s) ^ (~s & (unsigned short)0x8000);
}

// the logit of a key (inverse of the order map), as fp32
__device__ __forceinline__ float key_logit(uint32_t key) {
  const uint32_t hi = key & 0xffff0000u;
  const uint32_t bits = (hi & 0x80000000u) ? (hi ^ 0x80000000u) : (0u - hi);
  return __builtin_bit_cast(float, bits);
}

__device__ __forceinline__ uint32_t umed3(uint32_t a, uint32_t b, uint32_t c) {
  return max(min(a, b), min(max(a, b), c));
}

template <int KP>
__device__ __forceinline__ void sort_bitonic_desc(uint32_t (&m)[KP]) {
#pragma unroll
  for (int d = KP / 2; d >= 1; d /= 2)
#pragma unroll
    for (int i = 0; i < KP; ++i)
      if ((i & d) == 0) {
        const uint32_t hi = max(m[i], m[i + d]), lo = min(m[i], m[i + d]);
        m[i] = hi;
        m[i + d] = lo;
      }
}

template <int KP, int L>
__global__ __launch_bounds__(256) void moe_topk_softmax_kernel(MoeArgs a) {
  const int lane = threadIdx.x & 63;
  const int s = lane % L;                                    // this lane's share of the experts
  const long t = ((long)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / L) + lane / L;
  const bool live = t < a.num_tokens;
  const int per = (a.num_experts + L - 1) / L;
  const int e0 = s * per, e1 = min(e0 + per, a.num_experts);

  uint32_t top[KP];                                          // descending; 0 is below every key
#pragma unroll
  for (int i = 0; i < KP; ++i) top[i] = 0u;
  auto insert = [&](uint32_t key) {                          // top KP of the list and the key
#pragma unroll
    for (int i = KP - 1; i >= 1; --i) top[i] = umed3(top[i - 1], top[i], key);
    top[0] = max(top[0], key);
  };
  if (live) {
    const uint16_t* row = a.logits + t * a.num_experts;
    if (a.num_experts % (8 * L) == 0) {
      // whole 16-byte chunks (8 logits) per lane, all loads issued first
      const int nch = per / 8;                               // 1 .. 8 (the launch keeps E <= 64 L)
      u32x4 ch[8];
#pragma unroll
      for (int c = 0; c < 8; ++c)
        if (c < nch) ch[c] = *reinterpret_cast<const u32x4*>(row + e0 + 8 * c);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        if (c >= nch) break;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t idx = 0xffffu - (uint32_t)(e0 + 8 * c + 2 * w);
          const uint32_t k2 = __builtin_bit_cast(uint32_t, order_hi_pair(ch[c][w]));
          insert((k2 << 16) | idx);
          insert((k2 & 0xffff0000u) | (idx - 1));
        }
      }
    } else {
      for (int e = e0; e < e1; ++e) insert(order_key((uint32_t)row[e] << 16, 0xffffu - (uint32_t)e));
    }
  }
  // merge the L lists of the token's lanes (every lane takes part: the
  // exchanges stay inside each L-lane group)
#pragma unroll
  for (int m = 1; m < L; m <<= 1) {
    uint32_t other[KP];
#pragma unroll
    for (int i = 0; i < KP; ++i) other[i] = shfl_xor_u32(top[i], m);
#pragma unroll
    for (int i = 0; i < KP; ++i) top[i] = max(top[i], other[KP - 1 - i]);
    sort_bitonic_desc<KP>(top);
  }
  if (!live || s >= a.top_k) return;
  // softmax over the K selected logits (each lane sums them itself); lane s
  // writes entries s, s + L, ...
  const float l0 = key_logit(top[0]);
  float ex[KP];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    ex[i] = i < a.top_k ? exp2_hw((key_logit(top[i]) - l0) * kLog2e) : 0.f;
    sum += ex[i];
  }
#pragma unroll
  for (int i = 0; i < KP; ++i) {
    if (i % L != s || i >= a.top_k) continue;
    a.topk_idx[t * a.top_k + i] = 0xffff - (int)(top[i] & 0xffffu);
    a.topk_w[t * a.top_k + i] = to_bf16_bits(ex[i] / sum);
  }
}

}  // namespace

template <int L>
static hipError_t launch_lanes(const MoeArgs& a, hipStream_t stream) {
  const int per_block = 4 * (64 / L);                       // tokens per workgroup of four waves
  const dim3 grid((unsigned)((a.num_tokens + per_block - 1) / per_block)), block(256);
  if (a.top_k <= 1) hipLaunchKernelGGL((moe_topk_softmax_kernel<1, L>), grid, block, 0, stream, a);
  else if (a.top_k <= 2) hipLaunchKernelGGL((moe_topk_softmax_kernel<2, L>), grid, block, 0, stream, a);
  else if (a.top_k <= 4) hipLaunchKernelGGL((moe_topk_softmax_kernel<4, L>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((moe_topk_softmax_kernel<8, L>), grid, block, 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_moe_topk_softmax(const MoeArgs& a, hipStream_t stream) {
  if (a.num_tokens <= 0) return hipSuccess;
  // four lanes per token (one exchange level fewer) while a lane's share
  // stays whole 16-byte chunks within the register budget, else eight
  if (a.num_experts % 32 == 0 && a.num_experts <= 256) return launch_lanes<4>(a, stream);
  return launch_lanes<8>(a, stream);
}

}  // namespace sinkattn
