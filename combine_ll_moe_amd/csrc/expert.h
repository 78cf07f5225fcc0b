// Expert-side helpers: the per-expert counts of a set (low halves of its
// signal words) as an exclusive prefix in LDS, and the expert owning a row
// of the flattened (expert, slot) order of the received messages.
//
// Receive row e * max_tokens + j holds expert e's j-th message (rocSHMEM
// example LL_MoE/LL_MoE_Buffers.hpp, struct LLMoEBuffer, dispatch receive
// buffer); the counts say how many of each expert's rows are filled.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "route.h"

namespace llmoe {

// Rounds of count loads for E experts (kSendBlock threads load one each per
// round); the prefix then has kSendBlock * rounds + 1 entries.
__host__ __device__ constexpr int count_rounds(int num_experts) {
  return num_experts <= kSendBlock ? 1 : num_experts <= 4 * kSendBlock ? 4 : 16;
}
__host__ __device__ constexpr uint32_t count_prefix_bytes(int num_experts) {
  return ((uint32_t)(kSendBlock * count_rounds(num_experts) + 1) * 4u + 15u) & ~15u;
}

// Exclusive prefix of the counts (low halves of the signal words, each
// taken as at most max_tokens) into pre[0..E], pre[E] = total rows.
// ROUNDS * kSendBlock >= E. Thread tid loads experts tid + r * kSendBlock
// (coalesced, all loads issued before any is used), the counts go to LDS,
// then thread tid sums the contiguous run [tid * ROUNDS, (tid + 1) * ROUNDS)
// and a workgroup scan of the run sums gives each run its base.
template <int ROUNDS>
__device__ __forceinline__ void count_prefix(const unsigned long long* sig, int E, int max_tokens,
                                             uint32_t* pre, uint32_t* wave_sum) {
  const int tid = threadIdx.x;
  uint32_t c[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int e = tid + r * kSendBlock;
    const uint64_t w = __hip_atomic_load(sig + (e < E ? e : E - 1), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t n = (uint32_t)w;
    c[r] = e < E ? (n < (uint32_t)max_tokens ? n : (uint32_t)max_tokens) : 0u;
  }
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) pre[tid + r * kSendBlock] = c[r];
  __syncthreads();
  uint32_t run[ROUNDS];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) {
    run[i] = sum;
    sum += pre[tid * ROUNDS + i];
  }
  // inclusive scan of the run sums within the wavefront, then across waves
  const int lane = tid & (kWave - 1);
  uint32_t incl = sum;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint32_t o = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += o;
  }
  if (lane == kWave - 1) wave_sum[tid / kWave] = incl;
  __syncthreads();
  uint32_t base = incl - sum;
  for (int w = 0; w < tid / kWave; ++w) base += wave_sum[w];
#pragma unroll
  for (int i = 0; i < ROUNDS; ++i) pre[tid * ROUNDS + i] = base + run[i];
  if (tid == kSendBlock - 1) pre[kSendBlock * ROUNDS] = base + sum;
  __syncthreads();
}

// Expert of flattened row r: the largest e < E with pre[e] <= r (an expert
// with no rows has pre[e] == pre[e + 1], so it is never the answer for a
// row below pre[E]).
__device__ __forceinline__ int expert_of_row(const uint32_t* pre, int E, uint32_t r) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}


// count_prefix for any num_experts <= kSendMaxExperts; returns the total
// (the sum of the counts as taken). All threads of the workgroup call it.
__device__ __forceinline__ uint32_t load_count_prefix(const unsigned long long* sig, int E,
                                                      int max_tokens, uint32_t* pre,
                                                      uint32_t* wave_sum) {
  const int rounds = count_rounds(E);
  if (rounds == 1)
    count_prefix<1>(sig, E, max_tokens, pre, wave_sum);
  else if (rounds == 4)
    count_prefix<4>(sig, E, max_tokens, pre, wave_sum);
  else
    count_prefix<kSendMaxExperts / kSendBlock>(sig, E, max_tokens, pre, wave_sum);
  return pre[kSendBlock * rounds];
}

}  // namespace llmoe
