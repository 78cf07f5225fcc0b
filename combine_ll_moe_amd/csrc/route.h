// Device-side routing prologue shared by the dispatch and combine kernels.
//
// The receive buffer of a set holds num_experts * max_tokens message rows
// (rocSHMEM example LL_MoE/LL_MoE_Buffers.hpp, struct LLMoEBuffer, dispatch
// receive buffer); expert e owns rows [e * max_tokens, (e + 1) * max_tokens).
// A routed entry (t, k) goes to row e * max_tokens + slot(t, k), where
// slot(t, k) counts the earlier entries, in (t, k) order, that name the same
// expert: the entries of tokens before t, plus the picks of t itself before
// k. That is an exclusive prefix count per expert in ascending token order,
// which makes the slot order deterministic.
//
// Every workgroup that serves token t recomputes the slots of t from the
// routing table itself (no workspace, no second launch): the table is at
// most a few tens of KiB and stays in L2.
//  - Up to kHistExperts experts: a per-expert histogram of the earlier
//    tokens' entries in LDS, one LDS atomic per entry whatever topk is.
//  - More experts: a ballot per (entry, pick) over the earlier entries,
//    summed across the wavefronts in LDS.
// Loads are unconditional (indices clamped into the table, clamped lanes
// masked afterwards), so the compiler issues them back to back.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace llmoe {

constexpr int kWave = 64;
constexpr int kMaxWaves = 16;
constexpr int kHistExperts = 4096;

struct RouteShared {
  alignas(16) int expert[kMaxTopk];  // idx[t, k]
  alignas(16) int slot[kMaxTopk];    // slot(t, k), or -1 when the entry is masked
  int partial[kMaxWaves][kMaxTopk];
  int hist[kHistExperts];
};

// All threads of the workgroup must call this (it contains barriers).
// On return rs.expert[k] and rs.slot[k] hold token t's picks and slots for
// k < topk. blockDim.x must be a multiple of 64 and at most 1024, and
// 1 <= topk <= MAXK <= kMaxTopk.
template <int MAXK>
__device__ __forceinline__ void route_token(const int32_t* __restrict__ idx, int t, int topk,
                                            int num_experts, int max_tokens, RouteShared& rs) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int nthreads = blockDim.x;
  const int first = t * topk;  // entries of earlier tokens: [0, first)
  constexpr int kUnroll = 8;

  // the token's own picks (uniform; picks past topk repeat the last one and
  // are never used)
  int pick[MAXK];
#pragma unroll
  for (int k = 0; k < MAXK; ++k) pick[k] = idx[first + (k < topk ? k : topk - 1)];

  if (num_experts <= kHistExperts) {
    for (int e = tid; e < num_experts; e += nthreads) rs.hist[e] = 0;
    __syncthreads();
    const int last = first > 0 ? first - 1 : 0;
    for (int base = tid; base < first; base += nthreads * kUnroll) {
      int v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int p = base + u * nthreads;
        v[u] = idx[p < last ? p : last];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int p = base + u * nthreads;
        if (p < first && v[u] >= 0 && v[u] < num_experts) atomicAdd(&rs.hist[v[u]], 1);
      }
    }
    __syncthreads();
    if (tid < topk) {
      int e = pick[0];  // this thread's pick, and how often it came earlier in t
      int same = 0;
#pragma unroll
      for (int k = 0; k < MAXK; ++k) e = k == tid ? pick[k] : e;
#pragma unroll
      for (int k = 0; k < MAXK; ++k) same += (k < tid) & (pick[k] == e);
      const bool valid = e >= 0 && e < num_experts;
      const int s = valid ? rs.hist[e] + same : 0;
      rs.expert[tid] = e;
      rs.slot[tid] = valid && s < max_tokens ? s : -1;
    }
    __syncthreads();
    return;
  }

  // many experts: one ballot per (entry, pick); entry p counts for pick k
  // when it names the same expert and comes before (t, k): p < first + k
  const int end = first + topk;
  const int last = end - 1;
  int cnt[MAXK];  // wave-uniform
#pragma unroll
  for (int k = 0; k < MAXK; ++k) cnt[k] = 0;
  for (int base = wave * kWave; base < end; base += nthreads * kUnroll) {
    int v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = base + lane + u * nthreads;
      v[u] = idx[p < last ? p : last];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = base + lane + u * nthreads;
#pragma unroll
      for (int k = 0; k < MAXK; ++k) cnt[k] += __popcll(__ballot(v[u] == pick[k] && p < first + k));
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < MAXK; ++k) rs.partial[wave][k] = cnt[k];
  }
  if (tid == 0) {
#pragma unroll
    for (int k = 0; k < MAXK; ++k) rs.expert[k] = pick[k];
  }
  __syncthreads();
  if (tid < topk) {
    int s = 0;
    for (int w = 0; w < nthreads / kWave; ++w) s += rs.partial[w][tid];
    const int e = rs.expert[tid];
    const bool routed = e >= 0 && e < num_experts && s < max_tokens;
    rs.slot[tid] = routed ? s : -1;
  }
  __syncthreads();
}

}  // namespace llmoe
