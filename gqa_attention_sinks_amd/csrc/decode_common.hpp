// The work unit of a split decode launch (request, KV head, chunk), shared
// by the one-row and the several-row decode kernels.
#pragma once

#include "device_common.hpp"
#include "kernel_args.hpp"

namespace sinkattn {

// Requests ranked by KV length (longest first), so that the longest chunks
// start first and the short ones fill the tail; only for batches up to this
// size (the host passes the order with the launch, or every workgroup ranks
// the batch itself).  Padding entries of -1 never outrank a real request
// (kv_len >= 0).
constexpr int kRankMaxBatch = kPlanMaxBatch;
// Under a window up to this long every request's work is about the same, and
// ranking would only cost time.
constexpr int kRankMinWindow = kPlanMinWindow;

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
  if (a.planned) {   // the order, built on the host (any permutation gives the same results)
    u.b = a.order[r];
    u.n_k = a.kv_len[u.b];
    u.page_base = a.page_indptr[u.b];
    return u;
  }
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

}  // namespace sinkattn
