// Device-side helpers shared by the sink-attention kernels (gfx950 / CDNA4).
//
// Vector types for MFMA operands, bf16 packing, wavefront shuffles and the
// base-2 softmax constants.  The kernels work in the base-2 domain: scores are
// multiplied by sm_scale * log2(e) once, exponentials use the hardware exp2,
// and a head's sink enters as sink * log2(e) (the sink is already on the
// scaled-logit scale, so sm_scale never touches it).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kHeadDim = 64;
constexpr int kPageSize = 16;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Two fp32 -> two bf16 (round to nearest even) packed low/high in one dword.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

// Two fp32 -> two fp16 (round to nearest even) packed low/high in one dword.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// acc + lo + hi of a packed fp16 pair (v_dot2_f32_f16 against (1, 1)).  The
// softmax denominator is summed from the same rounded weights that feed the
// P.V matrix product, so numerator and denominator use identical weights.
__device__ __forceinline__ float add_f16x2(uint32_t packed, float acc) {
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), ones, acc, false);
}

// A dword holding two bf16 values -> the same two values as fp16 (exact for
// magnitudes in fp16's normal range, round to nearest otherwise).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t x) {
  const float lo = __builtin_bit_cast(float, x << 16);
  const float hi = __builtin_bit_cast(float, x & 0xffff0000u);
  return pack_f16x2(lo, hi);
}

// Fold the head's sink into a finished key-domain softmax state.
//
// The streaming softmax of the method keeps (m, d), seeded with (sink, 1), so
// after a set of keys with scaled logits s_j (base 2) it holds
//   m = max(sink, max_j s_j),  d = exp2(sink - m) + sum_j exp2(s_j - m).
// The kernels accumulate the same keys relative to the key maximum m_k
// (d_k = sum_j exp2(s_j - m_k), acc = sum_j exp2(s_j - m_k) v_j) so that the
// weights fed to the fp16 P.V product never underflow behind a large sink,
// and evaluate the seeded state once at the end:
//   m = max(sink, m_k),  d = exp2(sink - m) + exp2(m_k - m) * d_k,
//   out = acc * exp2(m_k - m) / d,  lse2 = m + log2(d)   (base 2).
// `sink2` is sink * log2(e), or -inf when this range carries no sink.
// Returns the factor that turns acc into out; writes lse2.
__device__ __forceinline__ float fold_sink(float sink2, float m_k, float d_k, float* lse2) {
  const float m = fmaxf(sink2, m_k);
  if (m == -__builtin_inff()) {          // no key and no sink
    *lse2 = m;
    return 0.f;
  }
  if (sink2 == __builtin_inff()) {       // infinite sink takes all the mass
    *lse2 = sink2;
    return 0.f;
  }
  const float wk = (m_k == m) ? 1.f : exp2_hw(m_k - m);
  const float ws = (sink2 == m) ? 1.f : exp2_hw(sink2 - m);
  const float d = ws + wk * d_k;
  *lse2 = m + log2_hw(d);
  return wk / d;
}

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Cross-lane exchange inside a 64-wide wavefront (through the LDS crossbar;
// touches no LDS memory).
__device__ __forceinline__ float shfl_xor_f32(float v, int mask) {
  const int lane = __lane_id();
  const int src = lane ^ mask;
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, v)));
}

// Byte-select of two dwords (v_perm_b32): result byte i = byte sel_i of
// {hi:lo} where bytes 0-3 come from lo and 4-7 from hi.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

}  // namespace sinkattn
