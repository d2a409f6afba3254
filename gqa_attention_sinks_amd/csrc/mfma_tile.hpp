// 32x32 MFMA tile helpers shared by the prefill and the verify decode: the
// LDS layout of a staged [key][64 dims] tile, the per-lane offsets of the
// K-operand and transposed V-operand reads, and the fp16 weights of a 32-key
// half tile.
//
// Score layout (v_mfma_f32_32x32x16, S^T = K . Q^T): element i of a lane's
// accumulator is key 8*(i/4) + 4*(lane/32) + i%4 of the 32-key half against
// column lane%32 of the 32-column block.
#pragma once

#include "device_common.hpp"

namespace sinkattn {

// Byte offset of 16-byte chunk `chunk` of key row `key` in a staged tile
// ([key][64 dims], 128 bytes a row).  The chunk position is XORed with a
// function of key bits 1-3 chosen so that the three access patterns of the
// kernel are conflict-free on the 64 four-byte LDS banks: the K operand reads
// (16 lanes per cycle on 16 consecutive keys), the transposing V reads (32
// lanes per cycle on 4 consecutive keys x 4 chunks) and the staging stores.
__device__ __forceinline__ uint32_t tile_swizzle(int key, int chunk) {
  const int a = (key >> 1) & 7;
  return key * 128 + ((chunk ^ (a ^ ((a & 1) << 2))) << 4);
}

// LDS pointer from a byte address in the workgroup's LDS (no null check).
template <typename T>
__device__ __forceinline__ __attribute__((address_space(3))) T* lds_at(uint32_t addr) {
  return (__attribute__((address_space(3))) T*)(size_t)addr;
}

// Per-lane byte offsets inside one staged tile, computed once; the key-block
// parts of each read (+32 keys, +16 keys) are constants in the offset field.
struct TileLanes {
  uint32_t k[4];      // K operand of MFMA step kstep: key r32, chunk 2*kstep + half
  uint32_t v[2][2];   // V^T operand, dims block db, keys kq (lo) and kq + 8 (hi)
};

__device__ __forceinline__ TileLanes tile_lanes(int lane) {
  TileLanes t;
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int kstep = 0; kstep < 4; ++kstep) t.k[kstep] = tile_swizzle(r32, 2 * kstep + half);
  const int j16 = lane & 15;
  const int kq = 4 * half + (j16 >> 2);
#pragma unroll
  for (int db = 0; db < 2; ++db) {
    const int chunk = 4 * db + 2 * ((lane >> 4) & 1) + ((j16 & 3) >> 1);
    t.v[db][0] = tile_swizzle(kq, chunk) + 8 * (j16 & 1);
    t.v[db][1] = tile_swizzle(kq + 8, chunk) + 8 * (j16 & 1);
  }
  return t;
}

// fp16 weights of one 32-key half of a tile against the reference m (base 2),
// packed as P^T operands (pop[rb][hh] covers keys 16*hh .. 16*hh+15 of the
// half, in the key order of the score accumulator), and this lane's share of
// each row's weight sum.  The sum is taken over the same rounded fp16 weights
// that feed the P.V product, with a tree of packed fp16 adds (two lanes of
// eight weights each, 2^-11 relative rounding per level) finished in fp32: the
// packed fp16 dot instruction would occupy the matrix pipe.  A sum that
// overflows fp16 comes out as +inf, which the caller's limit check catches.
// Weights of scores 2j and 2j+1 of row block rb, packed.
__device__ __forceinline__ void weight_pair(const f32x16 (&s)[2], const float (&m)[2], float c,
                                            int rb, int j, f16x2 (&h)[2][8]) {
  const float lo = exp2_hw(__builtin_fmaf(s[rb][2 * j], c, -m[rb]));
  const float hi = exp2_hw(__builtin_fmaf(s[rb][2 * j + 1], c, -m[rb]));
  h[rb][j] = __builtin_bit_cast(f16x2, pack_f16x2(lo, hi));
}

__device__ __forceinline__ void finish_weights(const f16x2 (&h)[2][8], f16x8 (&pop)[2][2],
                                               float (&tsum)[2]) {
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      pop[rb][hh] = __builtin_bit_cast(f16x8, u32x4{__builtin_bit_cast(uint32_t, h[rb][4 * hh]),
                                                    __builtin_bit_cast(uint32_t, h[rb][4 * hh + 1]),
                                                    __builtin_bit_cast(uint32_t, h[rb][4 * hh + 2]),
                                                    __builtin_bit_cast(uint32_t, h[rb][4 * hh + 3])});
    const f16x2 t = ((h[rb][0] + h[rb][1]) + (h[rb][2] + h[rb][3])) +
                    ((h[rb][4] + h[rb][5]) + (h[rb][6] + h[rb][7]));
    tsum[rb] = (float)t[0] + (float)t[1];
  }
}

__device__ __forceinline__ void half_weights(const f32x16 (&s)[2], const float (&m)[2], float c,
                                             f16x8 (&pop)[2][2], float (&tsum)[2]) {
  f16x2 h[2][8];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int j = 0; j < 8; ++j) weight_pair(s, m, c, rb, j, h);
  finish_weights(h, pop, tsum);
}

}  // namespace sinkattn
