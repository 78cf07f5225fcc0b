// Device-side routing prologue shared by the dispatch and combine kernels.
//
// The receive buffer of a set holds num_experts * max_tokens message rows
// (rocSHMEM example LL_MoE_Buffers.hpp, struct LLMoEBuffer, dispatch receive
// buffer); expert e owns rows [e * max_tokens, (e + 1) * max_tokens). A
// routed entry (t, k) goes to row e * max_tokens + slot(t, k), where
// slot(t, k) counts the earlier entries, in (t, k) order, that name the same
// expert. That is an exclusive prefix count per expert in ascending token
// order, which makes the slot order deterministic.
//
// Every workgroup that serves token t recomputes the K slots of t from the
// routing table itself: it scans the table up to t and counts matches per
// pick with per-lane counters, then reduces them across the wavefront and
// the workgroup. The table is at most a few tens of KiB and stays in L2, so
// the redundant scan costs L2 reads instead of a second launch or a
// workspace.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace llmoe {

constexpr int kWave = 64;
constexpr int kMaxWaves = 16;

struct RouteShared {
  int expert[kMaxTopk];  // idx[t, k]
  int slot[kMaxTopk];    // slot(t, k), or -1 when the entry is masked
  int partial[kMaxWaves][kMaxTopk];
};

// All threads of the workgroup must call this (it contains barriers).
// On return rs.expert[k] and rs.slot[k] hold token t's picks and slots for
// k < topk. blockDim.x must be a multiple of 64 and at most 1024, and
// topk <= MAXK <= kMaxTopk.
template <int MAXK>
__device__ __forceinline__ void route_token(const int32_t* __restrict__ idx, int t, int topk,
                                            int num_experts, int max_tokens, RouteShared& rs) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int nthreads = blockDim.x;
  const int64_t first = (int64_t)t * topk;  // entries of earlier tokens: [0, first)
  const int64_t end = first + topk;

  if (tid < topk) rs.expert[tid] = idx[first + tid];
  __syncthreads();

  int pick[MAXK];
  int cnt[MAXK];  // wave-uniform
#pragma unroll
  for (int k = 0; k < MAXK; ++k) {
    pick[k] = k < topk ? rs.expert[k] : INT32_MIN;
    cnt[k] = 0;
  }

  // Entry p counts for pick k when it names the same expert and comes
  // before (t, k): p < first + k. Each lane loads eight entries per round
  // (independent loads, all in flight together); a ballot per (entry, pick)
  // turns the 64 comparisons of a wavefront into one scalar popcount. The
  // round count is the same for every lane of the workgroup.
  constexpr int kUnroll = 8;
  for (int64_t base = (int64_t)wave * kWave; base < end; base += (int64_t)nthreads * kUnroll) {
    int v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t p = base + lane + (int64_t)u * nthreads;
      v[u] = p < end ? idx[p] : INT32_MIN + 1;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t p = base + lane + (int64_t)u * nthreads;
#pragma unroll
      for (int k = 0; k < MAXK; ++k)
        if (k < topk) cnt[k] += __popcll(__ballot(v[u] == pick[k] && p < first + k));
    }
  }

#pragma unroll
  for (int k = 0; k < MAXK; ++k)
    if (k < topk && lane == 0) rs.partial[wave][k] = cnt[k];
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
