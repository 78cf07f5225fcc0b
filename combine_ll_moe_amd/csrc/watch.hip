// A concurrent reader of a dispatch's signal words, for tests of the
// publish order: the counts are raised only after the messages they count
// are visible at device scope (mscclpp.h, the put-then-signal contract above
// struct mscclppDevConn: the receiver reads data only after it has seen the
// signal). Run on another stream while the dispatch runs. Workgroup b owns
// the experts e = b, b + G, ... (G workgroups) and repeatedly
//   1. loads its experts' counts with acquire semantics at device scope,
//   2. looks at those experts' receive rows that the routing says will be
//      filled, and counts those whose header names a token routed to the
//      expert and whose sampled payload words equal that token's row of x,
//   3. records a violation for every expert whose acquired count exceeds
//      the rows it found.
// A workgroup stops once its acquired counts add up to its experts' routed
// messages, or after max_passes passes, so every workgroup ends. A row
// written but not yet counted may or may not be found; only a count ahead
// of its rows is wrong.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ll_moe.h"
#include "ll_moe_diag.h"
#include "layout.h"

namespace llmoe {

namespace {

struct WatchParams {
  const unsigned long long* sig;   // signal words of set q
  const uint8_t* recv;             // receive buffer of set q
  const uint32_t* x;               // bf16 [num_tokens, hidden] as dwords
  const int32_t* idx;              // int32 [num_tokens, topk]
  int num_tokens;
  int max_tokens;
  int hidden;
  int num_experts;
  int topk;
  uint32_t msg_bytes;
  int max_passes;
  long long* report;               // int64 [4]
};

constexpr int kWatchMaxExperts = 2048;
constexpr int kWatchGroups = 64;
constexpr int kOwned = kWatchMaxExperts / kWatchGroups;  // experts per workgroup, at most
constexpr int kWatchBlock = 256;
constexpr int kPayloadSamples = 4;

__device__ __forceinline__ uint32_t load_coherent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void __launch_bounds__(kWatchBlock) watch_kernel(const WatchParams P) {
  __shared__ int cnt[kOwned];     // messages owned expert i will receive
  __shared__ int first[kOwned];   // running sum of cnt: i's first row in the walk
  __shared__ int pub[kOwned];     // count acquired in this pass
  __shared__ int found[kOwned];   // rows found complete in this pass
  __shared__ long long total[2];
  __shared__ int violations;
  const int tid = threadIdx.x;
  const int E = P.num_experts;
  const int K = P.topk;
  const int G = gridDim.x;
  const int b = blockIdx.x;
  const int owned = b < E ? (E - 1 - b) / G + 1 : 0;  // experts b, b + G, ... below E

  // the routing, as a count per owned expert (valid entries, at most max_tokens)
  for (int i = tid; i < kOwned; i += kWatchBlock) cnt[i] = 0;
  if (tid == 0) {
    total[0] = total[1] = 0;
    violations = 0;
  }
  __syncthreads();
  for (int j = tid; j < P.num_tokens * K; j += kWatchBlock) {
    const int e = P.idx[j];
    if (e >= 0 && e < E && e % G == b) atomicAdd(&cnt[e / G], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < owned; ++i) {
      const int c = cnt[i] < P.max_tokens ? cnt[i] : P.max_tokens;
      cnt[i] = c;
      first[i] = run;
      run += c;
    }
    total[1] = run;  // rows to expect; reset below, before pass 1 adds into it
  }
  __syncthreads();
  const long long expected = total[1];
  const int rows = (int)expected;
  __syncthreads();
  if (tid == 0) total[1] = 0;

  const int words = P.hidden / 2;  // payload dwords of a bf16 message
  int partial = 0;
  int pass = 0;
  long long seen = 0;
  while (pass < P.max_passes) {  // uniform
    // 1. acquire the counts
    if (tid < owned) {
      const unsigned long long v = __hip_atomic_load(P.sig + b + tid * G, __ATOMIC_ACQUIRE,
                                                     __HIP_MEMORY_SCOPE_AGENT);
      pub[tid] = (int)v;
      found[tid] = 0;
      atomicAdd(reinterpret_cast<unsigned long long*>(&total[pass & 1]), v);
    }
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");

    // 2. every expected row of the owned experts
    for (int r = tid; r < rows; r += kWatchBlock) {
      // the last i with first[i] <= r: an expert with no rows shares its
      // successor's first, so the last one of equal firsts has rows, and r
      // lies among them
      int i = 0;
      while (i + 1 < owned && first[i + 1] <= r) ++i;
      const int e = b + i * G;
      const int j = r - first[i];
      const uint32_t* row = reinterpret_cast<const uint32_t*>(
          P.recv + ((uint64_t)e * (uint64_t)P.max_tokens + (uint64_t)j) * P.msg_bytes);
      uint32_t got[kPayloadSamples + 1];
      got[0] = load_coherent(row);
#pragma unroll
      for (int s = 0; s < kPayloadSamples; ++s)
        got[s + 1] = load_coherent(row + 1 + (uint64_t)(words - 1) * s / (kPayloadSamples - 1));
      const int t = (int)got[0];
      bool ok = t >= 0 && t < P.num_tokens;
      if (ok) {
        bool routed = false;
        for (int k = 0; k < K; ++k) routed = routed || P.idx[(uint64_t)t * K + k] == e;
        ok = routed;
      }
      if (ok) {
        const uint32_t* xr = P.x + (uint64_t)t * words;
#pragma unroll
        for (int s = 0; s < kPayloadSamples; ++s)
          ok = ok && got[s + 1] == xr[(uint64_t)(words - 1) * s / (kPayloadSamples - 1)];
      }
      if (ok) atomicAdd(&found[i], 1);
    }
    __syncthreads();

    // 3. a count ahead of its rows is a violation
    if (tid < owned && pub[tid] > found[tid]) atomicAdd(&violations, 1);
    seen = total[pass & 1];
    __syncthreads();
    if (tid == 0) total[pass & 1] = 0;  // the next pass adds into the other word
    ++pass;
    if (seen > 0 && seen < expected) ++partial;
    if (seen >= expected) break;
  }
  __syncthreads();
  if (tid == 0) {
    atomicMax(reinterpret_cast<unsigned long long*>(P.report), (unsigned long long)pass);
    atomicAdd(reinterpret_cast<unsigned long long*>(P.report + 1), (unsigned long long)partial);
    atomicAdd(reinterpret_cast<unsigned long long*>(P.report + 2), (unsigned long long)violations);
    atomicAdd(reinterpret_cast<unsigned long long*>(P.report + 3), (unsigned long long)seen);
  }
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

}  // namespace
}  // namespace llmoe

using namespace llmoe;

extern "C" int ll_moe_diag_watch(const void* layout, int max_tokens, int num_tokens, int hidden,
                                 int num_experts, int topk, int parity, const void* x,
                                 const int32_t* topk_idx, int max_passes, long long* report,
                                 hipStream_t stream) {
  Layout L;
  if (parity != 0 && parity != 1) return LL_MOE_INVALID_ARGUMENT;
  if (!make_layout(max_tokens, hidden, num_experts, kBf16, &L)) return LL_MOE_INVALID_ARGUMENT;
  if (num_tokens < 0 || num_tokens > max_tokens || hidden % 8 != 0) return LL_MOE_INVALID_ARGUMENT;
  if (topk < 1 || topk > num_experts || topk > LL_MOE_MAX_TOPK) return LL_MOE_INVALID_ARGUMENT;
  if (num_experts > kWatchMaxExperts || max_passes < 1) return LL_MOE_INVALID_ARGUMENT;
  if ((int64_t)max_tokens * topk > INT32_MAX) return LL_MOE_INVALID_ARGUMENT;
  if (!layout || !report || !aligned(layout, 16) || !aligned(report, 8))
    return LL_MOE_INVALID_ARGUMENT;
  if (num_tokens > 0 && (!x || !topk_idx || !aligned(x, 16) || !aligned(topk_idx, 4)))
    return LL_MOE_INVALID_ARGUMENT;
  const uint8_t* base = static_cast<const uint8_t*>(layout);
  WatchParams p;
  p.sig = reinterpret_cast<const unsigned long long*>(base + L.sig_off(parity));
  p.recv = base + L.recv_off(parity);
  p.x = static_cast<const uint32_t*>(x);
  p.idx = topk_idx;
  p.num_tokens = num_tokens;
  p.max_tokens = max_tokens;
  p.hidden = hidden;
  p.num_experts = num_experts;
  p.topk = topk;
  p.msg_bytes = (uint32_t)L.dispatch_msg;
  p.max_passes = max_passes;
  p.report = report;
  const int groups = num_experts < kWatchGroups ? num_experts : kWatchGroups;
  watch_kernel<<<groups, kWatchBlock, 0, stream>>>(p);
  return hipGetLastError() == hipSuccess ? LL_MOE_SUCCESS : LL_MOE_HIP_ERROR;
}
